// dca_launch.hpp - internal host-side launchers (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dca {

constexpr int kPrefillTileKeys = 64;  // key rows per prefill K/V tile

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// RoPE cos/sin table [npos][D/2] of double2 (cos, sin), all in fp64.
hipError_t launch_rope_table(double2* table, int npos, int D, double base, hipStream_t st);

// dca_rope_remap kernel (dtype 0 = fp32, 1 = bf16).
hipError_t launch_rope_remap(const void* x, void* out, int64_t B, int64_t L, int64_t H, int64_t D,
                             int64_t pos0, int map, int c, int w, double base, int dtype,
                             hipStream_t st);

// Key rotation into head-major krot [B, Hkv, Lp, D] (+ optional BSHD copy):
// key j is turned to position (j / kdiv) mod kmod (DCA: kdiv 1, kmod s;
// SelfExtend neighbor keys: kdiv 1, grouped keys: kdiv G, kmod unbounded).
// For bf16 with vt non-null, also the tiled, key-permuted V transpose
// vt [B, Hkv, Lp/64, D, 64].
hipError_t launch_kv_prep(const void* k, const void* v, const double2* table, void* krot, void* vt,
                          void* k_rot_out, int64_t B, int64_t L, int64_t Lp, int64_t Hkv, int64_t D,
                          int kdiv, int kmod, int dtype, hipStream_t st);

// Position maps of the prefill kernels.
enum PosMap : int {
  kMapDCA = 0,         // chunk relation: intra / successive / inter queries, keys at j mod s
  kMapSelfExtend = 1,  // neighbor (i - j < W): plain positions; grouped: keys j/G,
                       // queries i/G + W - W/G
};
// SelfExtend pair classes (the order the kernels visit them in).
constexpr int kSeGrouped = 0;
constexpr int kSeNeighbor = 1;

struct PrefillArgs {
  const void* q;       // [B, L, Hq, D] raw
  const void* krot;    // [B, Hkv, Lp, D] rotated keys (DCA: at j mod s; SelfExtend: at j)
  const void* krot2;   // SelfExtend only: keys at floor(j / G); null for DCA
  const void* vt;      // bf16: [B, Hkv, Lp/64, D, 64]; fp32: raw v [B, L, Hkv, D]
  const double2* table; // [npos, D/2] (cos, sin) in fp64
  void* o;             // [B, L, Hq, D]
  float* lse;          // [B, Hq, L] or null
  int B, L, Lp, Hq, Hkv, D, c, w, s;
  int map;             // PosMap
  int se_group, se_window;  // SelfExtend G and W
  float sm_scale;
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
};

// Split plan shared by the workspace query and the launcher.
void decode_plan(int64_t B, int64_t kv_len, int64_t Hq, int64_t Hkv, int dtype, int* keys_per_split,
                 int* nsplit);
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t st);

}  // namespace dca
