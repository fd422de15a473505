// prefill.hip - DCA causal prefill attention kernels for gfx950.
//
// What is computed ("Dual-Chunk Attention: Training-Free 100k+ Context
// Guide", sections "The Architecture", "Intra-Chunk Attention", "Inter-Chunk
// Attention", "Successive Chunk Smoothing" and "Flash-DCA"): for query i and
// key j <= i the score is sm_scale * <R_{P_q} q_i, R_{j mod s} k_j>, where P_q
// is one of three query positions picked by the chunk relation of (i, j).  The
// softmax over j is merged tile by tile (online max / sum), so no L x L matrix
// exists.  When the chunk size is a multiple of the tile sizes every (query
// tile, key tile) pair has one relation, and a tile costs exactly what a plain
// flash-attention tile costs; otherwise the key tiles near the rows' chunks are
// cut at the chunk boundaries into "virtual tiles" of one relation each.
//
// One bf16 kernel, the two-group "ping-pong" kernel below, serves every map
// (DCA with any chunk size and query offset, SelfExtend, the guide's coarse /
// fine map); fp32 inputs take a plain VALU kernel.  The bf16 kernel:
//   * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = the
//     wave's 32 rotated queries held in registers.  In the 32x32 output layout
//     each lane owns one query column, so the row max / sum need a single
//     cross-half exchange.
//   * O^T += V^T * P^T on the same MFMA: A = V^T rows from LDS (pre-transposed
//     and key-permuted by the prep pass), B = the probabilities straight from
//     the S^T registers.
//   * K and V^T tiles are double-buffered in LDS, filled by direct
//     global->LDS buffer loads (no staging registers); rows padded by 16 bytes
//     make the MFMA fragment reads bank-conflict free with immediate offsets.
//   * The query variant lives in registers and is re-made (rotate raw Q with the
//     fp32 cos/sin table) only when the tile relation changes: inter ->
//     successive -> intra, at most three times per row, and not at all for
//     inter -> successive where both positions are c - 1.
//   * Online softmax in the log2 domain with a lazy rescale.
//   * Workgroups are ordered longest causal row first, and, when B*Hkv is a
//     multiple of 8, mapped so that each XCD (workgroup id mod 8) serves whole
//     GQA groups and their K/V stay in that XCD's L2.
#include <type_traits>

#include "dca_common.hpp"
#include "dca_launch.hpp"

namespace dca {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNoMax = -1.0e30f;  // running-max sentinel (finite)

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// s_waitcnt vmcnt(0): this wave's global loads (including the direct-to-LDS
// ones) have landed.  Encoding: vmcnt 0, expcnt 7, lgkmcnt 15.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- bf16 ping-pong kernel ------------------------------------------------------
// One workgroup = 8 waves = 256 query rows of one head; key tiles of
// TK = 64 * NSUB keys (128 when the chunk size allows: half the phase
// barriers per key, 2-3 % faster than 64).  Waves 0-3 (group 0) and 4-7
// (group 1) share the four SIMDs one-to-one and alternate, phase by phase,
// between
//   X(t): O^T += V(t-1)^T P(t-1)^T, then S^T(t) = K(t) Q^T    (TK/2 MFMAs)
//   Y(t): mask, exp, P(t) -> bf16, row sums, lazy rescale     (VALU)
// with group 1 one phase behind group 0, so each SIMD has one wave feeding the
// matrix core while the other runs the softmax (the hardware co-issues them;
// measured 4% faster than four independent waves per workgroup, and raising
// the MFMA wave's priority made it slower).  Phases end at a workgroup
// barrier.  K(t+1) and V(t) are loaded straight into LDS by group 0, one
// load every few MFMAs of its phase 2t, and waited for at the end of phase
// 2t+1; K and V are each double-buffered.  The softmax row sums add fp32
// probabilities with plain VALU adds (the bf16 dot2 instructions wait for the
// matrix pipe and would queue behind the other group's MFMAs).  With s a
// multiple of TK (and query offsets multiples of 32) every 32-row wave block
// lies in one chunk and every key tile in one chunk, so a (wave, tile) pair has
// a single relation (MAP kMapDCA).  Otherwise (kMapDCASplit) key tiles are cut
// at the chunk boundaries near the workgroup's rows and each lane picks its
// own query variant.
// Maximum of a lane's 32 scores as a tree of max3 (depth 4), so the wave is
// not held up by a 16-deep dependency chain.
__device__ inline float max32(const f32x16 (&x)[2]) {
  float t[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int a = 3 * i, b = a + 1, c = a + 2;
    t[i] = fmaxf(fmaxf(x[a >> 4][a & 15], x[b >> 4][b & 15]), x[c >> 4][c & 15]);
  }
  t[10] = fmaxf(x[1][14], x[1][15]);
  const float u0 = fmaxf(fmaxf(t[0], t[1]), t[2]), u1 = fmaxf(fmaxf(t[3], t[4]), t[5]);
  const float u2 = fmaxf(fmaxf(t[6], t[7]), t[8]), u3 = fmaxf(t[9], t[10]);
  return fmaxf(fmaxf(u0, u1), fmaxf(u2, u3));
}

constexpr int PP_BR = 256;

// LDS of the two-group kernel for key tiles of TK = 64 * NSUB keys: K rows
// (padded), then the V tile as NSUB sub-tiles of 64 keys, each [D][64]
// transposed exactly as the V layout in HBM holds it (padded rows); two
// buffers of each.
template <int D, int NSUB>
struct PPSmem {
  static constexpr int TK = 64 * NSUB;
  static constexpr int KROW = D * 2 + 16;
  static constexpr int VROW = 64 * 2 + 16;
  static constexpr int KBYTES = TK * KROW;
  static constexpr int VSUB = D * VROW;
  static constexpr int VBYTES = NSUB * VSUB;
  static constexpr int KPIECES = KBYTES / 1024;
  static constexpr int VPIECES = VSUB / 1024;   // per sub-tile
  static constexpr int TOTAL = 2 * (KBYTES + VBYTES);
  static_assert(KBYTES % 1024 == 0 && VSUB % 1024 == 0, "tiles must be whole 1 KiB pieces");
};

// Row max over the 32 * NSUB scores a lane holds.
template <int NSUB>
__device__ inline float max_tile(const f32x16 (&x)[2 * NSUB]) {
  if constexpr (NSUB == 1) {
    return max32(x);
  } else {
    const f32x16 lo[2] = {x[0], x[1]}, hi[2] = {x[2], x[3]};
    return fmaxf(max32(lo), max32(hi));
  }
}
constexpr float kSumLimit = 256.0f;  // per-lane probability sum that forces a rescale
// Word 3 of a raw buffer descriptor on gfx9-family parts (gfx950): 32-bit
// data format, no swizzle, offsets bounded by the record count in word 2.
constexpr int kBufferWord3 = 0x00020000;

// End of a phase: every LDS read of this wave has returned, then the
// workgroup barrier.  Written as asm (with a compiler memory clobber) so the
// compiler adds no wait on the direct-to-LDS loads still in flight, whose
// data is only needed two phases later.
// The scheduling barriers keep the compiler from moving any instruction
// across the phase boundary: MFMAs of an X phase sunk into the next phase
// would wait behind the other group's MFMA chain on the shared matrix pipe,
// and the softmax that needs their results with them.
__device__ inline void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, int MAP, int NSUB>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_pp_kernel(PrefillArgs a, int nqt, int xcd_map, float scale_log2) {
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  using SM = PPSmem<D, NSUB>;
  constexpr int TK = SM::TK;   // keys per tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];
  // LDS: K buffers 0/1 then V buffers 0/1.
  constexpr int KB0 = 0, VB0 = 2 * SM::KBYTES;

  // ---- work item (longest causal rows first, XCD-aware GQA grouping) ----------
  const int wg = blockIdx.x;
  int qt_rank, b, hq;
  const int G = a.Hq / a.Hkv;
  if (xcd_map) {
    const int xcd = wg & 7, k = wg >> 3;
    const int per_rank = (a.B * a.Hkv / 8) * G;
    qt_rank = k / per_rank;
    const int rem = k - qt_rank * per_rank;
    const int slot = (rem / G) * 8 + xcd;
    b = slot / a.Hkv;
    hq = (slot - b * a.Hkv) * G + rem % G;
  } else {
    const int bh = a.B * a.Hq;
    qt_rank = wg / bh;
    const int rem = wg - qt_rank * bh;
    b = rem / a.Hq;
    hq = rem - b * a.Hq;
  }
  const int qt = nqt - 1 - qt_rank;
  // This sequence's query rows sit at positions q0 .. q0 + nrows - 1 and see
  // the keys [0, q0 + nrows).  (DCA here needs q0 % 32 == 0: every wave
  // block inside one chunk.)
  int q0 = 0, nrows = a.L;
  if (a.per_seq) {
    q0 = a.seq_q0[b];
    nrows = a.seq_len[b];
  }
  if (qt * PP_BR >= nrows) return;   // whole workgroup, before any barrier
  const int64_t bg = (int64_t)b * a.Hkv + hq / G;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;
  const int hh = lane >> 5, ql = lane & 31;
  const int L = q0 + nrows, s = a.s, c = a.c;
  const int i0 = q0 + qt * PP_BR;
  const int i_lo = i0 + wave * 32;
  const int qrow = i_lo + ql;
  const int nq = i_lo / s;                 // the wave's 32 rows share one chunk (not for kMapDCASplit)
  // kMapDCASplit (any chunk size and query offset): a wave's 32 rows may span
  // a chunk boundary, so each lane takes the chunk of its own row.
  const int nq_l = MAP == kMapDCASplit ? qrow / s : nq;
  const int rq_l = qrow - nq_l * s;
  const int nkt = min(i0 + PP_BR - 1, L - 1) / TK + 1;

  // ---- order in which key tiles are visited ("virtual tiles" t) -------------
  // DCA: key tiles 0 .. nkt-1; a (wave, tile) pair has one chunk relation.
  // SelfExtend: first the tiles holding grouped pairs of this workgroup's rows
  // (j <= i - W), then those holding neighbor pairs (i - W < j <= i).  Tiles on
  // the window edge are visited twice, each time with the other class masked;
  // the class is the same for the whole workgroup, and selects the key
  // rotation staged and the query variant used.
  // Coarse / fine: the same two passes, split by key rotation.  First every
  // tile of a chunk at least two before the workgroup's last chunk (scaled
  // keys, inter query), then every tile from the chunk before its first chunk
  // on (plain keys; intra or successive query, chosen per wave).  A wave
  // whose relation to a tile belongs to the other pass sees it fully masked.
  // (A workgroup's 256 rows can span several chunks, so the key rotation
  // cannot follow one wave's relation: every wave stages part of each tile.)
  // DCA split map: key tiles cut at the chunk boundaries n s with
  // n >= split_nmin that fall inside a tile.  On the two sides of such a
  // boundary some row of this workgroup (whose lowest chunk is i0 / s) sees
  // different relations; older boundaries separate chunks that are both at
  // least two behind every row (inter on both sides) and are left uncut.  A
  // virtual tile then holds keys of one relation per row, so each lane can
  // take its own query variant.
  int n_gr = 0, nb_begin = 0, nvt = nkt, split_nmin = 1;
  if constexpr (MAP == kMapDCASplit) {
    const int key_last = min(i0 + PP_BR - 1, L - 1);
    split_nmin = max(i0 / s - 1, 1);
    const int n_hi = key_last / s;
    if (n_hi >= split_nmin) {
      const int m = TK / min(s & -s, TK);   // n s is a multiple of TK iff m divides n
      nvt = nkt + (n_hi - split_nmin + 1) - (n_hi / m - (split_nmin - 1) / m);
    }
  } else if constexpr (MAP == kMapSelfExtend) {
    const int W = a.se_window;
    const int i_top = min(i0 + PP_BR - 1, L - 1);
    n_gr = i_top >= W ? (i_top - W) / TK + 1 : 0;
    nb_begin = max(i0 - W + 1, 0) / TK;
    nvt = n_gr + (W > 0 ? nkt - nb_begin : 0);
  } else if constexpr (MAP == kMapCoarseFine) {
    const int c_first = i0 / s, c_last = min(i0 + PP_BR - 1, L - 1) / s;
    n_gr = c_last >= 2 ? (c_last - 1) * (s / TK) : 0;
    nb_begin = max(c_first - 1, 0) * (s / TK);
    nvt = n_gr + nkt - nb_begin;
  }
  auto tile_of = [&](int t) __attribute__((always_inline)) {
    if constexpr (MAP != kMapDCA) return t < n_gr ? t : nb_begin + (t - n_gr);
    return t;
  };
  // The query variant of virtual tile t for this wave.  Coarse / fine plain
  // pass: intra (0) or successive (1) by the wave's chunk distance, clamped
  // for masked tiles so the variant only moves inter -> successive -> intra.
  auto class_of = [&](int t) __attribute__((always_inline)) {
    if constexpr (MAP == kMapSelfExtend) return t < n_gr ? kSeGrouped : kSeNeighbor;
    if constexpr (MAP == kMapCoarseFine) return t < n_gr ? 2 : min(max(nq - (tile_of(t) * TK) / s, 0), 1);
    return min(nq - (t * TK) / s, 2);
  };
  // Coarse / fine: does this wave keep virtual tile t at all (else p = 0)?
  auto cf_keep = [&](int t) __attribute__((always_inline)) {
    const int rho = nq - (tile_of(t) * TK) / s;
    return t < n_gr ? rho >= 2 : (rho == 0 || rho == 1);
  };
  // A virtual tile: its index t (LDS buffer parity), its key tile, the keys
  // [lo, hi] it covers and (split map) the chunk of its first key.  The split
  // map's tiles are made one after the other from where the previous ended.
  struct VTile {
    int t, tile, lo, hi, nk;
  };
  auto vt_make = [&](int t) __attribute__((always_inline)) {
    VTile v;
    v.t = t;
    v.tile = tile_of(t);
    v.lo = v.tile * TK;
    v.hi = v.lo + TK - 1;
    v.nk = 0;
    return v;
  };
  auto vt_split = [&](int t, int start) __attribute__((always_inline)) {
    VTile v;
    v.t = t;
    v.tile = start / TK;
    v.nk = start / s;
    v.lo = start;
    const int tile_end = v.tile * TK + TK - 1;
    const int cut = max(v.nk + 1, split_nmin) * s;   // the next boundary that is cut
    v.hi = cut <= tile_end ? cut - 1 : tile_end;
    return v;
  };
  auto vt_first = [&]() __attribute__((always_inline)) {
    if constexpr (MAP == kMapDCASplit) return vt_split(0, 0);
    else return vt_make(0);
  };
  auto vt_next = [&](const VTile& v) __attribute__((always_inline)) {
    if constexpr (MAP == kMapDCASplit) return vt_split(v.t + 1, v.hi + 1);
    else return vt_make(v.t + 1);
  };

  const int64_t qoff = (int64_t)b * a.q_rows + (qrow - q0);   // row in q / o
  const uint16_t* qsrc = (const uint16_t*)a.q + (qoff * a.Hq + hq) * D;
  const uint16_t* kbase = (const uint16_t*)a.krot + bg * (int64_t)a.Lp * D;
  const uint16_t* vbase = (const uint16_t*)a.vt + bg * (int64_t)a.Lp * D;

  bf16x8 qf[NDS];
  // The query variant of class cls: the raw query turned by the (cos, sin)
  // of its query position, read from the fp32 frequency-major table (element
  // (P, k) at P * tab_ps + k * tab_ks): the 32 consecutive positions of a
  // wave read each frequency as 256 contiguous bytes.  A lane's 32 pairs and
  // its raw query fit in registers at once, so all its loads are in flight
  // together, and the rotation costs 4 fp32 operations per pair (fp64 needs
  // about 10 at the same per-instruction rate, beside the other group's
  // softmax on the same SIMD).  Rounding the angles and the rotation to fp32
  // moves a query by a few 2^-24, far below its bf16 rounding.  Rows past the
  // end get zero queries.
  auto load_q = [&](int cls) __attribute__((always_inline)) {
    if (qrow < L) {
      int64_t P;
      if constexpr (MAP == kMapCoarseFine)   // real positions: one table entry per (variant, row)
        P = (int64_t)cls * a.L + qrow;
      else if constexpr (MAP == kMapSelfExtend)
        P = cls == kSeNeighbor ? qrow : se_query_pos_grouped(qrow, a.se_group, a.se_window);
      else
        P = query_pos(cls, rq_l, s, c);
      const float2* ft = a.ftable + P * a.tab_ps + (int64_t)(hh * 8) * a.tab_ks;
      uint4 u[NDS];
      float2 tv[NDS / 2][8];
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds) {
        u[ds] = *(const uint4*)(qsrc + ds * 16 + hh * 8);
        u[ds + NDS / 2] = *(const uint4*)(qsrc + (ds + NDS / 2) * 16 + hh * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) tv[ds][e] = ft[(int64_t)(ds * 16 + e) * a.tab_ks];
      }
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds) {
        float x1[8], x2[8], y1[8], y2[8];
        unpack_bf16x8(u[ds], x1);
        unpack_bf16x8(u[ds + NDS / 2], x2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float cs = tv[ds][e].x, sn = tv[ds][e].y;
          y1[e] = fmaf(x1[e], cs, -(x2[e] * sn));
          y2[e] = fmaf(x2[e], cs, x1[e] * sn);
        }
        qf[ds] = as_bf16x8(pack_bf16x8(y1));
        qf[ds + NDS / 2] = as_bf16x8(pack_bf16x8(y2));
      }
    } else {
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) qf[ds] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  };

  // ---- direct-to-LDS staging ----------------------------------------------------
  // Group 0's four waves issue every 1-KiB piece of the tiles: K(t+1) and V(t)
  // are spread through the MFMA chain of their X(t) phase, one load every few
  // MFMAs.  (Issued at once by all eight waves at the start of a tile, the 70
  // loads of a 128-key tile queued in the load path for 700-1250 cycles and
  // held up the start of that phase for both groups.)  A wave with one piece
  // fewer than the others issues its last piece twice (the same bytes to the
  // same place), so every wave's chain has the same shape.
  constexpr int KPW = (SM::KPIECES + 3) / 4;   // K loads per group-0 wave and tile
  constexpr int VPW = (SM::VPIECES + 3) / 4;   // V loads per sub-tile and group-0 wave
  constexpr int NLOAD = KPW + NSUB * VPW;      // loads per group-0 wave and tile
  const int lw = wave & 3;
  auto kpiece = [&](int i) __attribute__((always_inline)) {
    const int p = lw + 4 * i;
    return p < SM::KPIECES ? p : p - 4;
  };
  auto vpiece = [&](int i) __attribute__((always_inline)) {
    const int p = lw + 4 * i;
    return p < SM::VPIECES ? p : p - 4;
  };
  // Per-lane source offsets inside a tile (K below 32 KiB, a V sub-tile
  // below 16 KiB), two 16-bit offsets per register.
  static_assert(SM::KPIECES * 1024 <= 65536 && SM::VSUB <= 65536, "offsets must fit in 16 bits");
  uint32_t koff2[(KPW + 1) / 2], voff2[(VPW + 1) / 2];
#pragma unroll
  for (int i = 0; i < (KPW + 1) / 2; ++i) koff2[i] = 0;
#pragma unroll
  for (int i = 0; i < (VPW + 1) / 2; ++i) voff2[i] = 0;
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int byte = kpiece(i) * 1024 + lane * 16;
    const int row = byte / SM::KROW, w = byte % SM::KROW;
    koff2[i >> 1] |= (uint32_t)(row * D * 2 + (w < D * 2 ? w : 0)) << (16 * (i & 1));
  }
#pragma unroll
  for (int i = 0; i < VPW; ++i) {
    const int byte = vpiece(i) * 1024 + lane * 16;
    const int row = byte / SM::VROW, w = byte % SM::VROW;
    voff2[i >> 1] |= (uint32_t)(row * 64 * 2 + (w < 64 * 2 ? w : 0)) << (16 * (i & 1));
  }
  auto koff = [&](int i) __attribute__((always_inline)) { return (koff2[i >> 1] >> (16 * (i & 1))) & 0xffffu; };
  auto voff = [&](int i) __attribute__((always_inline)) { return (voff2[i >> 1] >> (16 * (i & 1))) & 0xffffu; };
  // K/V tiles go straight to LDS through buffer loads (MUBUF with the lds
  // bit).  The descriptor covers this head's Lp rows exactly; a load past them
  // (the K tile after the last one, which the last X phase issues and nothing
  // reads) returns zeros.  The FLAT form of the same DMA would make the
  // compiler wait for every outstanding LDS read (lgkmcnt(0)) while it is in
  // flight.
  const uint32_t head_bytes = (uint32_t)((int64_t)a.Lp * D * 2);
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, head_bytes, kBufferWord3);
  // SelfExtend: grouped keys (at floor(j / G)); coarse / fine: scaled keys
  __amdgpu_buffer_rsrc_t krsrc2 = krsrc;
  if constexpr (MAP != kMapDCA)
    krsrc2 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint16_t*)a.krot2 + bg * (int64_t)a.Lp * D), (short)0, head_bytes, kBufferWord3);
  // K piece slot i of virtual tile vk
  auto load_k = [&](const VTile& vk, int i) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)vk.tile * (uint32_t)(TK * D * 2);
    __amdgpu_buffer_rsrc_t rs = krsrc;
    if constexpr (MAP == kMapSelfExtend)
      if (class_of(vk.t) == kSeGrouped) rs = krsrc2;
    if constexpr (MAP == kMapCoarseFine)
      if (vk.t < n_gr) rs = krsrc2;   // the scaled-key pass (same for every wave)
    uint8_t* dst = smem + KB0 + (vk.t & 1) * SM::KBYTES + kpiece(i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, (int)koff(i),
                                             (int)soff, 0, 0);
  };
  // V piece slot i of sub-tile sub of virtual tile v (NSUB consecutive 64-key
  // tiles of the HBM layout)
  auto load_v = [&](const VTile& v, int sub, int i) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)(v.tile * NSUB + sub) * (uint32_t)(64 * D * 2);
    uint8_t* dst = smem + VB0 + (v.t & 1) * SM::VBYTES + sub * SM::VSUB + vpiece(i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (__attribute__((address_space(3))) void*)dst, 16, (int)voff(i),
                                             (int)soff, 0, 0);
  };
  // load slot s of X(t) (v = t, vn = t + 1): K(t+1) pieces first, then V(t)
  auto load_slot = [&](const VTile& v, const VTile& vn, int s) __attribute__((always_inline)) {
    if (s < KPW)
      load_k(vn, s);
    else
      load_v(v, (s - KPW) / VPW, (s - KPW) % VPW);
  };
  const int kfrag = ql * SM::KROW + hh * 16;
  const int vfrag = ql * SM::VROW + hh * 16;
  // LDS offset of the PV operand fragment for 16-key group g4 and 32-dim block db
  auto voffs = [](int g4, int db) constexpr { return (g4 >> 2) * SM::VSUB + db * 32 * SM::VROW + (g4 & 3) * 32; };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
  f32x16 sacc[2 * NSUB];
  bf16x8 pf[4 * NSUB];
  float m_run = kNoMax, l_run = 0.f;
  int cur_cls = -1;

  auto do_pv = [&](int t) {
    const uint8_t* vb = smem + VB0 + (t & 1) * SM::VBYTES + vfrag;
#pragma unroll
    for (int g4 = 0; g4 < 4 * NSUB; ++g4)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 vf = *(const bf16x8*)(vb + voffs(g4, db));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[g4], oacc[db], 0, 0, 0);
      }
  };
  auto do_qk = [&](int t) {
    const uint8_t* kb = smem + KB0 + (t & 1) * SM::KBYTES + kfrag;
#pragma unroll
    for (int kb2 = 0; kb2 < 2 * NSUB; ++kb2)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb2][v] = 0.f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kb2 = 0; kb2 < 2 * NSUB; ++kb2) {
        const bf16x8 kf = *(const bf16x8*)(kb + kb2 * 32 * SM::KROW + ds * 32);
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], sacc[kb2], 0, 0, 0);
      }
  };
  auto do_softmax = [&](const VTile& v) {
    const int t = v.t;
    const int j0 = v.tile * TK;
    // Keys this lane keeps: [lo, hi].  DCA: the causal prefix.  SelfExtend:
    // grouped j <= i - W, neighbor i - W < j <= i.  The mask is applied only
    // when the tile is not wholly inside every row's range.
    int lo = 0, hi = qrow;
    bool need = j0 + TK - 1 > i_lo;
    if constexpr (MAP == kMapSelfExtend) {
      const int W = a.se_window;
      if (class_of(t) == kSeGrouped) {
        hi = qrow - W;
        need = j0 + TK - 1 > i_lo - W;
      } else {
        lo = qrow - W + 1;
        need = need || j0 < i_lo + 32 - W;
      }
    }
    if constexpr (MAP == kMapCoarseFine) {
      if (!cf_keep(t)) {
        lo = 1;
        hi = 0;
        need = true;
      }
    }
    if constexpr (MAP == kMapDCASplit) {   // the virtual tile's keys only
      lo = v.lo;
      hi = min(v.hi, qrow);
      need = need || v.lo > j0 || v.hi < j0 + TK - 1;
    }
    if (need) {
      const int jb = j0 + hh * 4;
#pragma unroll
      for (int kb2 = 0; kb2 < 2 * NSUB; ++kb2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = jb + kb2 * 32 + (v >> 2) * 8 + (v & 3);
          sacc[kb2][v] = (j >= lo && j <= hi) ? sacc[kb2][v] : -INFINITY;
        }
    }
    // Probabilities against the running max first.  A lane whose 32 * NSUB
    // probabilities sum past 2^8 (or to inf on the first tile, where the
    // running max is the sentinel) sends the wave through the exact rescale:
    // the true max, the accumulator rescale and the exps again.  Every stored
    // probability is therefore at most 2^8 and O and l share one max.
    // The row sum adds the fp32 probabilities with plain VALU adds: the
    // bf16 dot2 instructions wait for the matrix pipe, so in the softmax phase
    // they would queue behind the other group's MFMAs (measured: a wave of
    // exp + dot2 runs fully serialised against an MFMA wave on its SIMD,
    // exp + add overlaps it).
    auto exps = [&]() {
      float lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g4 = 0; g4 < 4 * NSUB; ++g4) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[g4 >> 1][(g4 & 1) * 8 + e], scale_log2, -m_run));
          lsum[g4 & 3] += p[e];
        }
        pf[g4] = as_bf16x8(pack_bf16x8(p));
        // keeps the compiler from computing all 32 * NSUB exps before packing
        // any (their fp32 values would not fit in the register budget)
        asm volatile("" : "+v"(pf[g4]));
      }
      return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };
    float lt = exps();
    if (__any(!(lt <= kSumLimit))) {
      const float mnew = max_halves(max_tile<NSUB>(sacc)) * scale_log2;
      const float mn = fmaxf(m_run, mnew);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
      m_run = mn;
      lt = exps();
    }
    l_run += lt;
  };

  // The probabilities feed the next phase's PV product; without this the
  // compiler sinks their exps past the phase barrier, next to that use.
  auto pin_p = [&]() {
    asm volatile("" : "+v"(pf[0]), "+v"(pf[1]), "+v"(pf[2]), "+v"(pf[3]), "+v"(l_run));
    if constexpr (NSUB == 2) asm volatile("" : "+v"(pf[4]), "+v"(pf[5]), "+v"(pf[6]), "+v"(pf[7]));
  };

  // ---- phases ---------------------------------------------------------------
  // Both groups execute the same number of barriers; each runs its own loop
  // so every iteration is straight-line code.  Tiles past a wave's last row
  // are processed fully masked (p = 0) rather than skipped.
  // The query variant of virtual tile v, re-made when it changes.  Split map:
  // each lane's own class (rows of one wave can span a chunk boundary); the
  // wave re-makes its variants when any lane's class changes.
  // DCA: a row whose successive position min(s + r, c - 1) is already c - 1
  // (r >= w - 1) has the same successive and inter variant, so a wave whose
  // rows all have that property keeps its registers when the relation moves
  // from inter to successive.
  auto same_pos = [&](int c1, int c2) __attribute__((always_inline)) {
    return c2 >= 0 && query_pos(c1, rq_l, s, c) == query_pos(c2, rq_l, s, c);
  };
  auto prep_q = [&](const VTile& v) __attribute__((always_inline)) {
    if constexpr (MAP == kMapDCASplit) {
      const int cls = min(max(nq_l - v.nk, 0), 2);
      if (__any(cls != cur_cls)) {
        if (!__all(same_pos(cls, cur_cls))) load_q(cls);
        cur_cls = cls;
      }
    } else {
      const int cls = class_of(v.t);
      if (cls != cur_cls) {
        if (MAP != kMapDCA || !__all(same_pos(cls, cur_cls))) load_q(cls);
        cur_cls = cls;
      }
    }
  };
  // X(t) for 0 < t < nvt: PV(t-1) then QK(t) as one chain of 32 MFMAs whose
  // LDS operands are read NPRE fragments ahead (a ring of registers), so each
  // MFMA waits only for the oldest read in flight.
  // With LOADS (group 0), the NLOAD load slots are spread evenly over the
  // NX MFMAs: slot floor(i NLOAD / NX) follows MFMA i where that value steps.
  auto x_full = [&](const VTile& v, const VTile& vn, auto loads) {
    constexpr bool LOADS = decltype(loads)::value;
    const int t = v.t;
    prep_q(v);
    constexpr int NKB = 2 * NSUB;   // 32-key blocks per tile
    constexpr int NPV = 4 * NSUB * NDB, NQK = NKB * NDS, NX = NPV + NQK, NPRE = 6;
    static_assert(NLOAD <= NX, "at most one load per MFMA");
    auto is_slot = [](int i) constexpr { return ((i + 1) * NLOAD) / NX > (i * NLOAD) / NX; };
    auto slot_of = [](int i) constexpr { return (i * NLOAD) / NX; };
    const uint8_t* vb = smem + VB0 + ((t - 1) & 1) * SM::VBYTES + vfrag;
    const uint8_t* kb = smem + KB0 + (t & 1) * SM::KBYTES + kfrag;
    auto frag = [&](int i) -> bf16x8 {
      if (i < NPV) {
        const int g4 = i / NDB, db = i % NDB;
        return *(const bf16x8*)(vb + voffs(g4, db));
      }
      const int ds = (i - NPV) / NKB, kb2 = (i - NPV) % NKB;
      return *(const bf16x8*)(kb + kb2 * 32 * SM::KROW + ds * 32);
    };
    bf16x8 ring[NPRE];
#pragma unroll
    for (int i = 0; i < NPRE; ++i) ring[i] = frag(i);
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb2][v] = 0.f;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const bf16x8 f = ring[i % NPRE];
      if (i + NPRE < NX) ring[i % NPRE] = frag(i + NPRE);
      if (i < NPV) {
        const int g4 = i / NDB, db = i % NDB;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[g4], oacc[db], 0, 0, 0);
      } else {
        const int ds = (i - NPV) / NKB, kb2 = (i - NPV) % NKB;
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[ds], sacc[kb2], 0, 0, 0);
      }
      if constexpr (LOADS)
        if (is_slot(i)) load_slot(v, vn, slot_of(i));
    }
    // Order: NPRE reads, then (MFMA, read[, load]) groups, then the last MFMAs.
#pragma unroll
    for (int i = 0; i < NPRE; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + NPRE < NX) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (LOADS && is_slot(i)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  };
  // Group 0 stages K(0) before the first barrier, then K(1) and V(0); from
  // then on K(t+1) and V(t) inside its X(t) phase.  It waits for its loads at
  // the end of the following Y phase, whose barrier makes them visible to
  // both groups before their next use.
  using kLoads = std::integral_constant<bool, true>;
  using kNoLoads = std::integral_constant<bool, false>;
  VTile vcur = vt_first(), vnxt = vt_next(vcur);
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < KPW; ++i) load_k(vcur, i);
  }
  wait_vmem();
  phase_barrier();
  // tile 0 (the first X phase has no PV; the last one, at t = nvt, has no QK)
  if (grp == 0) {
#pragma unroll
    for (int s2 = 0; s2 < NLOAD; ++s2) load_slot(vcur, vnxt, s2);
    prep_q(vcur);
    do_qk(0);
    phase_barrier();
    do_softmax(vcur);
    wait_vmem();
    phase_barrier();
    for (int t = 1; t < nvt; ++t) {
      vcur = vnxt;
      vnxt = vt_next(vnxt);
      x_full(vcur, vnxt, kLoads{});
      phase_barrier();
      do_softmax(vcur);
      wait_vmem();
      phase_barrier();
    }
    do_pv(nvt - 1);
    phase_barrier();
    phase_barrier();
  } else {
    // the first query variant's loads overlap group 0's K(0) loads
    prep_q(vcur);
    phase_barrier();
    do_qk(0);
    phase_barrier();
    VTile vprv = vcur;
    for (int t = 1; t < nvt; ++t) {
      vcur = vnxt;
      vnxt = vt_next(vnxt);
      do_softmax(vprv);
      pin_p();
      phase_barrier();
      x_full(vcur, vnxt, kNoLoads{});
      phase_barrier();
      vprv = vcur;
    }
    do_softmax(vprv);
    phase_barrier();
    do_pv(nvt - 1);
    phase_barrier();
  }

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = sum_halves(l_run);
  if (qrow < L) {
    const float inv = 1.f / l_tot;
    uint16_t* dst = (uint16_t*)a.o + (qoff * a.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int grp4 = 0; grp4 < 4; ++grp4) {
        uint2 wv;
        wv.x = pack_bf16x2(oacc[db][grp4 * 4] * inv, oacc[db][grp4 * 4 + 1] * inv);
        wv.y = pack_bf16x2(oacc[db][grp4 * 4 + 2] * inv, oacc[db][grp4 * 4 + 3] * inv);
        *(uint2*)(dst + db * 32 + grp4 * 8 + hh * 4) = wv;
      }
    if (hh == 0 && a.lse)
      a.lse[((int64_t)b * a.Hq + hq) * a.q_rows + (qrow - q0)] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// ---- fp32 kernel (VALU, exact-arithmetic path for fp32 inputs) ---------------------
// One workgroup = 16 query rows of one head; 16 lanes per row, 32-key tiles.
// Every pair picks its query variant (and, for SelfExtend, its key rotation)
// on its own.
constexpr int FBR = 16, FBC = 32;

template <int D, int MAP>
__global__ void __launch_bounds__(256) prefill_f32_kernel(PrefillArgs a) {
  constexpr int HALF = D / 2;
  constexpr int NO = D / 16;
  constexpr int NV = MAP == kMapSelfExtend ? 2 : 3;   // query variants
  __shared__ float qv[NV][D][FBR];
  __shared__ float ks[FBC][D + 1];
  // second key rotation: SelfExtend grouped keys / coarse-fine scaled keys
  __shared__ float ks2[MAP != kMapDCA ? FBC : 1][D + 1];
  __shared__ float vs[FBC][D];
  __shared__ float ps[FBR][FBC + 1];
  const int qt = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  int q0 = 0, nrows = a.L;   // this sequence's query rows: positions q0 .. q0 + nrows - 1
  if (a.per_seq) {
    q0 = a.seq_q0[b];
    nrows = a.seq_len[b];
  }
  if (qt * FBR >= nrows) return;   // whole workgroup, before any barrier
  const int L = q0 + nrows, s = a.s, c = a.c;
  const int G = a.Hq / a.Hkv, g = hq / G;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int tid = threadIdx.x;
  const int r = tid >> 4, kq = tid & 15;
  const int i0 = q0 + qt * FBR, i = i0 + r;
  const float* q = (const float*)a.q;
  const float* krot = (const float*)a.krot + bg * (int64_t)a.Lp * D;
  const float* krot2 = (const float*)a.krot2 + bg * (int64_t)a.Lp * D;   // SelfExtend only
  const float* vraw = (const float*)a.vt;
  const int W = a.se_window;

  for (int idx = tid; idx < FBR * HALF; idx += 256) {
    const int rr = idx / HALF, k = idx - rr * HALF;
    const int ii = i0 + rr;
    if (ii >= L) {   // padding rows: zero queries (their table position may not exist)
#pragma unroll
      for (int cls = 0; cls < NV; ++cls) qv[cls][k][rr] = qv[cls][k + HALF][rr] = 0.f;
      continue;
    }
    const float* src = q + (((int64_t)b * a.q_rows + (ii - q0)) * a.Hq + hq) * D;
    const float x1 = src[k], x2 = src[k + HALF];
    const int rqq = ii % s;
#pragma unroll
    for (int cls = 0; cls < NV; ++cls) {
      double2 t;
      if constexpr (MAP == kMapCoarseFine) {
        t = a.table[((int64_t)cls * a.L + ii) * a.tab_ps + k * a.tab_ks];
      } else {
        int P;
        if constexpr (MAP == kMapSelfExtend)
          P = cls == kSeNeighbor ? ii : se_query_pos_grouped(ii, a.se_group, W);
        else
          P = query_pos(cls, rqq, s, c);
        t = a.table[(int64_t)P * a.tab_ps + k * a.tab_ks];
      }
      qv[cls][k][rr] = (float)((double)x1 * t.x - (double)x2 * t.y);
      qv[cls][k + HALF][rr] = (float)((double)x2 * t.x + (double)x1 * t.y);
    }
  }
  float m = -INFINITY, l = 0.f, o[NO];
#pragma unroll
  for (int u = 0; u < NO; ++u) o[u] = 0.f;
  const int nq = i / s;
  const int last_key = min(i0 + FBR - 1, L - 1);
  const int nkt = last_key / FBC + 1;
  for (int kt = 0; kt < nkt; ++kt) {
    const int j0 = kt * FBC;
    __syncthreads();
    for (int idx = tid; idx < FBC * D; idx += 256) {
      const int row = idx / D, d = idx - row * D;
      const int j = j0 + row;
      ks[row][d] = krot[(int64_t)j * D + d];
      if constexpr (MAP != kMapDCA) ks2[row][d] = krot2[(int64_t)j * D + d];
      const int64_t crow = j < L ? cache_row(a.pg, a.v_rows, b, j) : 0;
      vs[row][d] = j >= L ? 0.f : (crow < 0 ? __builtin_nanf("") : vraw[(crow * a.Hkv + g) * D + d]);
    }
    __syncthreads();
    float sc[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = kq * 2 + e, j = j0 + key;
      if (j > i || j >= L) {
        sc[e] = -INFINITY;
      } else {
        float acc = 0.f;
        if constexpr (MAP == kMapSelfExtend) {
          const bool grouped = i - j >= W;
          const int cls = grouped ? kSeGrouped : kSeNeighbor;
          const float* kr = grouped ? ks2[key] : ks[key];
#pragma unroll 8
          for (int d = 0; d < D; ++d) acc = fmaf(qv[cls][d][r], kr[d], acc);
        } else {
          const int cls = min(nq - j / s, 2);
          const float* kr = (MAP == kMapCoarseFine && cls == 2) ? ks2[key] : ks[key];
#pragma unroll 8
          for (int d = 0; d < D; ++d) acc = fmaf(qv[cls][d][r], kr[d], acc);
        }
        sc[e] = acc * a.sm_scale;
      }
    }
    float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mn = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
    const float p0 = (sc[0] == -INFINITY) ? 0.f : expf(sc[0] - mn);
    const float p1 = (sc[1] == -INFINITY) ? 0.f : expf(sc[1] - mn);
    float psum = p0 + p1;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) psum += __shfl_xor(psum, off);
    l = l * alpha + psum;
    m = mn;
    ps[r][kq * 2] = p0;
    ps[r][kq * 2 + 1] = p1;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int d = kq + 16 * u;
      float acc = o[u] * alpha;
#pragma unroll 8
      for (int key = 0; key < FBC; ++key) acc = fmaf(ps[r][key], vs[key][d], acc);
      o[u] = acc;
    }
  }
  if (i < L) {
    float* dst = (float*)a.o + (((int64_t)b * a.q_rows + (i - q0)) * a.Hq + hq) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int u = 0; u < NO; ++u) dst[kq + 16 * u] = o[u] * inv;
    if (kq == 0 && a.lse) a.lse[((int64_t)b * a.Hq + hq) * a.q_rows + (i - q0)] = m + logf(l);
  }
}

}  // namespace

// The two-group kernel at one map and tile width, either head dim.
template <int MAP, int NSUB>
void launch_pp(const PrefillArgs& a, dim3 grid, int nqt, int xcd_map, float scale_log2, hipStream_t st) {
  if (a.D == 64)
    hipLaunchKernelGGL((prefill_bf16_pp_kernel<64, MAP, NSUB>), grid, dim3(512), 0, st, a, nqt, xcd_map, scale_log2);
  else
    hipLaunchKernelGGL((prefill_bf16_pp_kernel<128, MAP, NSUB>), grid, dim3(512), 0, st, a, nqt, xcd_map, scale_log2);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t st) {
  const int xcd_map = ((int64_t)a.B * a.Hkv) % 8 == 0 ? 1 : 0;
  const float scale_log2 = a.sm_scale * kLog2e;
  const int nqt = (a.q_rows + PP_BR - 1) / PP_BR;
  const dim3 grid((unsigned)((int64_t)nqt * a.B * a.Hq));
  // DCA runs the plain map when every 32-row wave block and every 64-key
  // tile lies inside one chunk (s a multiple of 64, query offsets multiples
  // of 32), else the split map.  128-key tiles (half the phase barriers per
  // key) whenever the chunk size allows them; the split map takes them when
  // chunks are long enough that the extra cut tiles are few.
  if (a.map == kMapSelfExtend) {
    launch_pp<kMapSelfExtend, 2>(a, grid, nqt, xcd_map, scale_log2, st);
  } else if (a.map == kMapCoarseFine) {
    if (a.s % 64 != 0) return hipErrorInvalidValue;   // needs chunk % 64 == 0 (host-checked)
    if (a.s % 128 == 0) launch_pp<kMapCoarseFine, 2>(a, grid, nqt, xcd_map, scale_log2, st);
    else launch_pp<kMapCoarseFine, 1>(a, grid, nqt, xcd_map, scale_log2, st);
  } else {
    bool aligned = a.s % 64 == 0;
    if (a.per_seq)
      for (int i = 0; i < a.B; ++i) aligned = aligned && a.seq_q0[i] % 32 == 0;
    if (aligned) {
      if (a.s % 128 == 0) launch_pp<kMapDCA, 2>(a, grid, nqt, xcd_map, scale_log2, st);
      else launch_pp<kMapDCA, 1>(a, grid, nqt, xcd_map, scale_log2, st);
    } else {
      if (a.s >= 256) launch_pp<kMapDCASplit, 2>(a, grid, nqt, xcd_map, scale_log2, st);
      else launch_pp<kMapDCASplit, 1>(a, grid, nqt, xcd_map, scale_log2, st);
    }
  }
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.q_rows + FBR - 1) / FBR), (unsigned)a.Hq, (unsigned)a.B);
  if (a.map == kMapSelfExtend) {
    if (a.D == 64)
      hipLaunchKernelGGL((prefill_f32_kernel<64, kMapSelfExtend>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_f32_kernel<128, kMapSelfExtend>), grid, dim3(256), 0, st, a);
  } else if (a.map == kMapCoarseFine) {
    if (a.D == 64)
      hipLaunchKernelGGL((prefill_f32_kernel<64, kMapCoarseFine>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_f32_kernel<128, kMapCoarseFine>), grid, dim3(256), 0, st, a);
  } else {
    if (a.D == 64)
      hipLaunchKernelGGL((prefill_f32_kernel<64, kMapDCA>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_f32_kernel<128, kMapDCA>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dca
