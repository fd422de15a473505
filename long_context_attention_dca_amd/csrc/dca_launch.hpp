// dca_launch.hpp - internal host-side launchers (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dca {

constexpr int kPrefillTileKeys = 64;  // keys per V tile of the prefill layout (and per prepare block)
constexpr int kPrefillRowAlign = 128; // key rows per head are padded to this (the widest key tile)
// Sequences whose own lengths / offsets one launch carries in its kernel
// arguments (ragged batches are launched in groups of at most this many).
constexpr int kMaxSeqGroup = 64;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// RoPE cos/sin table [npos][D/2] of double2 (cos, sin), all in fp64.
// kmajor: the frequency-major layout [D/2][npos] instead.
hipError_t launch_rope_table(double2* table, int npos, int D, double base, bool kmajor, hipStream_t st);
// The same angles rounded to fp32, frequency-major [D/2][npos] float2 (the bf16
// prefill kernel's DCA query rotations).
hipError_t launch_rope_table_f32(float2* table, int npos, int D, double base, hipStream_t st);
// theta_k = base^(-2k/D) for k < D/2, fp64 (for real-valued positions).
hipError_t launch_rope_theta(double* theta, int D, double base, hipStream_t st);
// Coarse / fine map: (cos, sin) of the three query positions of rows 0 .. L-1,
// frequency-major [D/2][3][L] double2, from theta (chunk C, 1 / kappa = inv_kappa).
hipError_t launch_cf_query_table(double2* tab, int L, int D, int C, double inv_kappa, const double* theta,
                                 hipStream_t st);
// The same, rounded to fp32 (the bf16 prefill kernel).
hipError_t launch_cf_query_table_f32(float2* tab, int L, int D, int C, double inv_kappa, const double* theta,
                                     hipStream_t st);

// dca_rope_remap kernel (dtype 0 = fp32, 1 = bf16).  map kRemapCoarseScaled
// (internal): the coarse / fine map's scaled key position, floor(p / c) *
// step + p mod c with step = C / kappa (w unused).
constexpr int kRemapCoarseScaled = 7;
hipError_t launch_rope_remap(const void* x, void* out, int64_t B, int64_t L, int64_t H, int64_t D,
                             int64_t pos0, int map, int c, int w, double base, int dtype,
                             hipStream_t st, double step = 0.0);

// Key rotation into head-major krot [B, Hkv, Lp, D] (+ optional BSHD copy):
// key j is turned to position (j / kdiv) mod kmod (DCA: kdiv 1, kmod s;
// SelfExtend neighbor keys: kdiv 1, grouped keys: kdiv G, kmod unbounded).
// With table == null the keys are already rotated (a KV cache) and are
// copied as they are.  For bf16 with vt non-null, also the tiled,
// key-permuted V transpose vt [B, Hkv, Lp/64, D, 64].  Rows at or past a
// sequence's valid length are written as zeros.
// A paged KV cache: k / v point at page pools [num_pages, page_size, Hkv, D];
// row j of sequence b is row j mod page_size of page bt[b * max_blocks +
// j / page_size].  bt null: the dense layout.
struct PagedKv {
  const int* bt;
  int page_size, max_blocks, num_pages;
};

struct KvPrepArgs {
  const void* k;        // [B, in_rows, Hkv, D]
  const void* v;        // [B, in_rows, Hkv, D]
  const double2* table; // rotation table, or null (copy)
  void* krot;
  void* vt;             // null: keys only
  void* k_rot_out;      // [B, in_rows, Hkv, D] copy of the rotated keys, or null
  int B, in_rows, L, Lp, Hkv, D, kdiv, kmod;
  int per_seq;          // 1: seq_len[b] valid rows per sequence (else L)
  int seq_len[kMaxSeqGroup];
  // pos_mode 1 (no cos/sin table): key j at floor(j / cf_chunk) * cf_step +
  // j mod cf_chunk, a real number, with cos/sin made in fp64 from theta
  // (cf_step = cf_chunk: plain positions; cf_chunk / kappa: coarse-scaled).
  int pos_mode;
  int cf_chunk;
  double cf_step;
  const double* theta;  // pos_mode 1: theta_k table [D/2]
  PagedKv pg;           // paged k / v (in_rows unused), or bt null
  // pos_mode 2 (bf16, table null): key j at (j / kdiv) mod kmod with its
  // cos / sin made in this kernel from base, exactly as launch_rope_table
  // makes them; the launch also writes that table rounded to fp32,
  // frequency-major ([D/2][table_rows]), to table_out (for the attention
  // kernel's query rotations).
  double base;
  float2* table_out;
  int table_rows;
};
hipError_t launch_kv_prep(const KvPrepArgs& a, int dtype, hipStream_t st);

// Position maps of the prefill kernels.
enum PosMap : int {
  kMapDCA = 0,         // chunk relation: intra / successive / inter queries, keys at j mod s
  kMapSelfExtend = 1,  // neighbor (i - j < W): plain positions; grouped: keys j/G,
                       // queries i/G + W - W/G
  kMapCoarseFine = 2,  // the DCA guide's own distances: chunk C (held in c and s),
                       // coarse chunk distance scaled by 1/kappa for pairs >= 2
                       // chunks apart, lambda ramp for adjacent chunks
  kMapDCASplit = 3,    // DCA when the chunk size is not a multiple of the key
                       // tile or query offsets are not multiples of 32 (kernel
                       // internal: key tiles cut at chunk boundaries, per-lane
                       // query variants); chosen by the launcher, never passed in
};
// SelfExtend pair classes (the order the kernels visit them in).
constexpr int kSeGrouped = 0;
constexpr int kSeNeighbor = 1;

struct PrefillArgs {
  const void* q;       // [B, L, Hq, D] raw
  const void* krot;    // [B, Hkv, Lp, D] rotated keys (DCA: at j mod s; SelfExtend: at j)
  const void* krot2;   // SelfExtend only: keys at floor(j / G); null for DCA
  const void* vt;      // bf16: [B, Hkv, Lp/64, D, 64]; fp32: raw v [B, L, Hkv, D]
  const double2* table; // fp32 kernel: (cos, sin) in fp64 of npos positions x D/2 frequencies; kMapCoarseFine:
                        // 3 L positions, the intra / successive / inter query positions of row i
                        // at cls * L + i
  // Element (position P, frequency k) is table[P * tab_ps + k * tab_ks]: row-major
  // (tab_ps = D/2, tab_ks = 1) or frequency-major (tab_ps = 1, tab_ks = npos).  The
  // frequency-major form lets a wave's 32 consecutive query positions read one
  // frequency's (cos, sin) as contiguous 512 bytes instead of 32 separate rows.
  int64_t tab_ps, tab_ks;
  // The bf16 kernel reads the angles rounded to fp32 (float2) here, with the
  // same strides; table is then unused.
  const float2* ftable;
  void* o;             // [B, L, Hq, D]
  float* lse;          // [B, Hq, L] or null
  int B, L, Lp, Hq, Hkv, D, c, w, s;
  int map;             // PosMap
  int se_group, se_window;  // SelfExtend G and W
  float sm_scale;
  // Query rows.  Whole prompts (per_seq 0): query row r of every sequence is
  // the token at position r, r < L, and q / o / lse hold q_rows = L rows.
  // Chunks (per_seq 1): sequence b's query row r is the token at position
  // seq_q0[b] + r for r < seq_len[b]; its keys are [0, seq_q0[b] + seq_len[b]);
  // q / o / lse hold q_rows rows per sequence.  L is then the largest key count.
  int q_rows;
  int per_seq;
  int seq_q0[kMaxSeqGroup];
  int seq_len[kMaxSeqGroup];
  int v_rows;          // fp32 kernels: rows per sequence of the raw V in vt
  PagedKv pg;           // fp32 kernels: raw V in a paged pool (v_rows unused), or bt null
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st);

struct DecodeArgs {
  const void* q;       // [B, Hq, D] raw
  const void* kc;      // [B, kv_len, Hkv, D] rotated at j mod s
  const void* vc;      // [B, kv_len, Hkv, D]
  void* o;             // [B, Hq, D]
  float* lse;          // [B, Hq] or null
  void* qv;            // workspace: [B, Hq, 3, D] rotated query variants (dtype)
  float* part_o;       // workspace: [B, Hq, NS, D]
  float* part_lse;     // workspace: [B, Hq, NS]  (log2 domain)
  int B, kv_len, Hq, Hkv, D, c, w, s;
  double base;
  float sm_scale;
  int keys_per_split;  // multiple of 32
  int nsplit;          // NS
  // Rows per sequence in the caches (the row stride; kv_len for a uniform
  // batch).  per_seq 1: sequence b uses seq_len[b] cached keys and its new
  // token sits at seq_len[b] - 1 (else every sequence uses kv_len).
  int cache_len;
  int per_seq;
  int seq_len[kMaxSeqGroup];
  // bf16 split kernel: waves are numbered flat over the real (sequence, unit,
  // key range) items; sequence b's waves start at wave_start[b] (set by the
  // launcher).
  int wave_start[kMaxSeqGroup + 1];
  PagedKv pg;          // kc / vc are page pools (cache_len unused), or bt null
  // Position map (PosMap).  SelfExtend and coarse / fine keep two key caches:
  // keys j < seg[b] (grouped, resp. two or more chunks before the query's)
  // are read from kc2, the others from kc; a key range may hold keys of
  // both.  DCA: seg[b] = 0, kc2 unused.  The query variants: DCA intra /
  // succ / inter; SelfExtend grouped / neighbor; coarse / fine intra / succ
  // / inter at real positions.
  int map;
  const void* kc2;
  int seg[kMaxSeqGroup];
  int se_group, se_window;
  double cf_inv_kappa;
};

// Split plan shared by the workspace queries and the launchers: kv holds the
// B sequences' cached key counts (host memory), or is null for B sequences
// of uniform_kv keys.
void decode_plan(const int64_t* kv, int64_t B, int64_t uniform_kv, int64_t Hq, int64_t Hkv, int dtype,
                 int* keys_per_split, int* nsplit);
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t st);

}  // namespace dca
