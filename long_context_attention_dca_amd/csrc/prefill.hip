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
// flash-attention tile costs; otherwise a straddling tile is processed once
// per relation it contains, with the other relations' pairs masked out.
//
// Two bf16 kernels share the tile math below: a two-group "ping-pong" kernel
// used whenever the chunk size is a multiple of 64 (every (wave, tile) pair
// has one relation), and a general kernel for any other chunk size.
//
// General bf16 kernel (one workgroup = 4 waves = 128 query rows of one head):
//   * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = the
//     wave's 32 rotated queries held in registers.  In the 32x32 output layout
//     each lane owns one query column, so the row max / sum need a single
//     cross-half exchange.
//   * O^T += V^T * P^T on the same MFMA: A = V^T rows from LDS (pre-transposed
//     and key-permuted by the prep pass), B = the probabilities straight from
//     the S^T registers.
//   * K and V^T tiles of 64 keys are double-buffered in LDS, filled by direct
//     global->LDS loads (no staging registers); rows padded by 16 bytes make
//     the MFMA fragment reads bank-conflict free with immediate offsets; one
//     barrier per tile.
//   * The query variant lives in registers and is re-made (rotate raw Q with the
//     cos/sin table) only when the tile relation changes: inter -> successive
//     -> intra, at most three times per workgroup on the fast path.
//   * Online softmax in the log2 domain; rescaling of the accumulator is skipped
//     while the running max grows by less than 8 (exact: O and l share the
//     stale max).
//   * Workgroups are ordered longest causal row first, and, when B*Hkv is a
//     multiple of 8, mapped so that each XCD (workgroup id mod 8) serves whole
//     GQA groups and their K/V stay in that XCD's L2.
#include "dca_common.hpp"
#include "dca_launch.hpp"

namespace dca {

namespace {

constexpr int BR = 128;  // query rows per workgroup (4 waves x 32)
constexpr int BC = kPrefillTileKeys;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;
constexpr float kNoMax = -1.0e30f;  // running-max sentinel (finite)

// LDS tiles.  Rows are padded by 16 bytes (K: 2D + 16, V^T: 2*64 + 16), which
// spreads the 16 rows a quarter-wave reads over all 64 banks, and keeps every
// fragment address of a tile a compile-time offset from one per-lane base.
// Both tiles are whole multiples of 1 KiB, the unit of a direct-to-LDS load.
template <int D>
struct Smem {
  static constexpr int KROW = D * 2 + 16;
  static constexpr int VROW = BC * 2 + 16;
  static constexpr int KBYTES = BC * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int KPIECES = KBYTES / 1024;
  static constexpr int VPIECES = VBYTES / 1024;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int TOTAL = 2 * STAGE;
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "tiles must be whole 1 KiB pieces");
};

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ inline bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }
__device__ constexpr bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};

// s_waitcnt vmcnt(0): this wave's global loads (including the direct-to-LDS
// ones) have landed.  Encoding: vmcnt 0, expcnt 7, lgkmcnt 15.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_kernel(PrefillArgs a, int nqt, int xcd_map, float scale_log2) {
  constexpr int NDS = D / 16;          // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;          // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<D>::TOTAL];

  // ---- work item ------------------------------------------------------------
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
  // the keys [0, q0 + nrows).
  int q0 = 0, nrows = a.L;
  if (a.per_seq) {
    q0 = a.seq_q0[b];
    nrows = a.seq_len[b];
  }
  if (qt * BR >= nrows) return;   // whole workgroup, before any barrier
  const int g = hq / G;
  const int64_t bg = (int64_t)b * a.Hkv + g;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, ql = lane & 31;
  const int L = q0 + nrows, s = a.s, c = a.c;
  const int i0 = q0 + qt * BR;
  const int qrow = i0 + wave * 32 + ql;
  const int i_lo = i0 + wave * 32;
  const int i_hi = min(i_lo + 31, L - 1);
  const bool wave_live = i_lo < L;
  const int n_lo = i_lo / s, n_hi = wave_live ? i_hi / s : 0;
  const int nq = qrow / s, rq = qrow - nq * s;
  const int last_key = min(i0 + BR - 1, L - 1);
  const int nkt = last_key / BC + 1;

  const int64_t qoff = (int64_t)b * a.q_rows + (qrow - q0);   // row in q / o
  const uint16_t* qsrc = (const uint16_t*)a.q + (qoff * a.Hq + hq) * D;
  const uint16_t* kbase = (const uint16_t*)a.krot + bg * (int64_t)a.Lp * D;
  const uint16_t* vbase = (const uint16_t*)a.vt + bg * (int64_t)a.Lp * D;

  // ---- query variant in registers (B operand of S^T = K Q^T) ------------------
  // Lane (query ql, half hh) holds dims d = ds*16 + hh*8 + e; the rotate-half
  // partner d + D/2 is in step ds + NDS/2 of the same lane.
  bf16x8 qf[NDS];
  auto load_q = [&](int cls) __attribute__((always_inline)) {
    const int P = query_pos(cls, rq, s, c);
    const double2* tb = a.table + (int64_t)P * (D / 2);
    if (qrow < L) {
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds) {
        const uint4 u1 = *(const uint4*)(qsrc + ds * 16 + hh * 8);
        const uint4 u2 = *(const uint4*)(qsrc + (ds + NDS / 2) * 16 + hh * 8);
        float x1[8], x2[8], y1[8], y2[8];
        unpack_bf16x8(u1, x1);
        unpack_bf16x8(u2, x2);
        // Rotation in fp64, one rounding to bf16 (through fp32).
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double2 t = tb[ds * 16 + hh * 8 + e];
          y1[e] = (float)((double)x1[e] * t.x - (double)x2[e] * t.y);
          y2[e] = (float)((double)x2[e] * t.x + (double)x1[e] * t.y);
        }
        qf[ds] = as_bf16x8(pack_bf16x8(y1));
        qf[ds + NDS / 2] = as_bf16x8(pack_bf16x8(y2));
      }
    } else {
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) qf[ds] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  };

  // ---- K / V^T staging: direct global -> LDS loads ----------------------------
  // global_load_lds_dwordx4 writes lane l's 16 bytes to LDS base + 16*l: a wave
  // fills one 1-KiB piece of the padded tile per instruction.  Each lane's
  // source offset inside a tile is the same for every tile, so it is computed
  // once; lanes that land on a row's 16-byte pad fetch that row's first chunk
  // (a valid address; the pad is never read).  Pieces go round-robin to waves.
  constexpr int KPW = (Smem<D>::KPIECES + 3) / 4;
  constexpr int VPW = (Smem<D>::VPIECES + 3) / 4;
  uint32_t koff[KPW], voff[VPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int byte = (wave + 4 * i) * 1024 + lane * 16;
    const int row = byte / Smem<D>::KROW, w = byte % Smem<D>::KROW;
    koff[i] = (uint32_t)(row * D * 2 + (w < D * 2 ? w : 0));
  }
#pragma unroll
  for (int i = 0; i < VPW; ++i) {
    const int byte = (wave + 4 * i) * 1024 + lane * 16;
    const int row = byte / Smem<D>::VROW, w = byte % Smem<D>::VROW;
    voff[i] = (uint32_t)(row * BC * 2 + (w < BC * 2 ? w : 0));
  }
  auto issue_tile = [&](int kt, int stage) {
    const uint8_t* ks = (const uint8_t*)(kbase + (int64_t)kt * BC * D);
    const uint8_t* vs = (const uint8_t*)(vbase + (int64_t)kt * BC * D);
    uint8_t* kb = smem + stage * Smem<D>::STAGE;
    uint8_t* vb = kb + Smem<D>::KBYTES;
#pragma unroll
    for (int i = 0; i < KPW; ++i)
      if (wave + 4 * i < Smem<D>::KPIECES)
        __builtin_amdgcn_global_load_lds((const void*)(ks + koff[i]),
                                         (__attribute__((address_space(3))) void*)(kb + (wave + 4 * i) * 1024),
                                         16, 0, 0);
#pragma unroll
    for (int i = 0; i < VPW; ++i)
      if (wave + 4 * i < Smem<D>::VPIECES)
        __builtin_amdgcn_global_load_lds((const void*)(vs + voff[i]),
                                         (__attribute__((address_space(3))) void*)(vb + (wave + 4 * i) * 1024),
                                         16, 0, 0);
  };
  // Per-lane fragment bases: K row (kb*32 + ql), V^T row (db*32 + ql); the
  // lane's half hh selects the second 16 bytes of each 32-byte k-step.
  const int kfrag = ql * Smem<D>::KROW + hh * 16;
  const int vfrag = Smem<D>::KBYTES + ql * Smem<D>::VROW + hh * 16;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
  // Running max (log2 domain).  The finite sentinel keeps rows that have seen
  // no unmasked key yet NaN-free: their p is exp2(-inf) = 0 and alpha is 1.
  float m_run = kNoMax, l_run = 0.f;
  int cur_cls = -1;

  issue_tile(0, 0);
  wait_vmem();
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nkt) issue_tile(kt + 1, stage ^ 1);
    const int j0 = kt * BC;
    if (wave_live && j0 <= i_hi) {
      // Chunk relations present among the unmasked pairs of this wave x tile.
      const int jmax = min(j0 + BC - 1, i_hi);
      const int rho_lo = max(n_lo - jmax / s, 0);
      const int rho_hi = n_hi - j0 / s;
      const int cls_lo = min(rho_lo, 2), cls_hi = min(rho_hi, 2);
      const bool straddle = cls_lo != cls_hi;
      const bool causal = j0 + BC - 1 > i_lo;
      // A tile whose pairs fall in several relations is processed once per
      // relation, with the other relations' pairs masked out; the online
      // softmax merges the pieces like ordinary tiles.
      for (int cls = cls_lo; cls <= cls_hi; ++cls) {
        if (cls != cur_cls) {
          load_q(cls);
          cur_cls = cls;
        }
        // The tile's LDS offset goes through an empty asm so the fragment
        // reads below are not hoisted out of this (rarely repeated) loop.
        int toff = stage * Smem<D>::STAGE;
        asm volatile("" : "+v"(toff));
        const uint8_t* kb = smem + toff + kfrag;
        const uint8_t* vb = smem + toff + vfrag;
        f32x16 sacc[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[0][v] = sacc[1][v] = 0.f;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const bf16x8 kf = *(const bf16x8*)(kb + kb2 * 32 * Smem<D>::KROW + ds * 32);
            sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], sacc[kb2], 0, 0, 0);
          }
        }
        if (causal || straddle) {
          // Keys this lane keeps: the causal prefix j <= qrow, intersected on a
          // straddling tile with the key range of relation `cls` for this row
          // (intra: chunk nq, successive: chunk nq-1, inter: chunks < nq-1).
          int lo = 0, hi = qrow;
          if (straddle) {
            lo = cls == 0 ? nq * s : (cls == 1 ? (nq - 1) * s : 0);
            hi = min(hi, cls == 0 ? qrow : (cls == 1 ? nq * s - 1 : (nq - 1) * s - 1));
          }
          const int jb = j0 + hh * 4;
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int j = jb + kb2 * 32 + (v >> 2) * 8 + (v & 3);
              sacc[kb2][v] = (j >= lo && j <= hi) ? sacc[kb2][v] : -INFINITY;
            }
        }

        // ---- online softmax (log2 domain) ----
        float mx = sacc[0][0];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb2][v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = mx * scale_log2;
        if (__any(mnew > m_run + kRescaleThreshold)) {
          const float mn = fmaxf(m_run, mnew);
          const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
          m_run = mn;
        }
        float lsum = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][u * 8 + e], scale_log2, -m_run));
            const uint4 pu = pack_bf16x8(p);
            // Row sum of the bf16-rounded probabilities (the values PV uses).
            lsum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pu.x), kOnes, lsum, false);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pu.y), kOnes, lsum, false);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pu.z), kOnes, lsum, false);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pu.w), kOnes, lsum, false);
            const bf16x8 pf = as_bf16x8(pu);
            // ---- O^T += V^T P^T for this 16-key group ----
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const bf16x8 vf = *(const bf16x8*)(vb + db * 32 * Smem<D>::VROW + (kb2 * 2 + u) * 32);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[db], 0, 0, 0);
            }
          }
        }
        l_run += lsum;
      }
    }
    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < L) {
    const float inv = 1.f / l_tot;
    uint16_t* dst = (uint16_t*)a.o + (qoff * a.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        uint2 wv;
        wv.x = pack_bf16x2(oacc[db][grp * 4] * inv, oacc[db][grp * 4 + 1] * inv);
        wv.y = pack_bf16x2(oacc[db][grp * 4 + 2] * inv, oacc[db][grp * 4 + 3] * inv);
        *(uint2*)(dst + db * 32 + grp * 8 + hh * 4) = wv;
      }
    if (hh == 0 && a.lse)
      a.lse[((int64_t)b * a.Hq + hq) * a.q_rows + (qrow - q0)] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// ---- bf16 ping-pong kernel (chunk size a multiple of 64) ------------------------
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
// barrier.  K(t+1) and V(t) are loaded straight into LDS at the
// start of phase 2t and waited for at the end of phase 2t+1; K and V are each
// double-buffered.  With s a multiple of TK every 32-row wave block lies in
// one chunk and every key tile in one chunk, so a (wave, tile) pair has a
// single relation and no straddle handling is needed.
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
__device__ inline void phase_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
  const int nq = i_lo / s;                 // the wave's 32 rows share one chunk
  const int rq = qrow - nq * s;
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
  int n_gr = 0, nb_begin = 0, nvt = nkt;
  if constexpr (MAP == kMapSelfExtend) {
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

  const int64_t qoff = (int64_t)b * a.q_rows + (qrow - q0);   // row in q / o
  const uint16_t* qsrc = (const uint16_t*)a.q + (qoff * a.Hq + hq) * D;
  const uint16_t* kbase = (const uint16_t*)a.krot + bg * (int64_t)a.Lp * D;
  const uint16_t* vbase = (const uint16_t*)a.vt + bg * (int64_t)a.Lp * D;

  bf16x8 qf[NDS];
  auto load_q = [&](int cls) __attribute__((always_inline)) {
    // this row's (cos, sin) row of the table, read only for rows < L
    const double2* tb;
    if constexpr (MAP == kMapCoarseFine) {   // real positions: one table row per (variant, row)
      tb = a.table + ((int64_t)cls * a.L + qrow) * (D / 2);
    } else {
      const int P = MAP == kMapSelfExtend
                        ? (cls == kSeNeighbor ? qrow : se_query_pos_grouped(qrow, a.se_group, a.se_window))
                        : query_pos(cls, rq, s, c);
      tb = a.table + (int64_t)P * (D / 2);
    }
    if (qrow < L) {
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds) {
        const uint4 u1 = *(const uint4*)(qsrc + ds * 16 + hh * 8);
        const uint4 u2 = *(const uint4*)(qsrc + (ds + NDS / 2) * 16 + hh * 8);
        float x1[8], x2[8], y1[8], y2[8];
        unpack_bf16x8(u1, x1);
        unpack_bf16x8(u2, x2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double2 t = tb[ds * 16 + hh * 8 + e];
          y1[e] = (float)((double)x1[e] * t.x - (double)x2[e] * t.y);
          y2[e] = (float)((double)x2[e] * t.x + (double)x1[e] * t.y);
        }
        qf[ds] = as_bf16x8(pack_bf16x8(y1));
        qf[ds + NDS / 2] = as_bf16x8(pack_bf16x8(y2));
      }
    } else {
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) qf[ds] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  };

  // ---- direct-to-LDS staging, 1-KiB pieces round-robin over the 8 waves -----
  constexpr int KPW = (SM::KPIECES + 7) / 8;
  constexpr int VPW = (SM::VPIECES + 7) / 8;
  uint32_t koff[KPW], voff[VPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int byte = (wave + 8 * i) * 1024 + lane * 16;
    const int row = byte / SM::KROW, w = byte % SM::KROW;
    koff[i] = (uint32_t)(row * D * 2 + (w < D * 2 ? w : 0));
  }
#pragma unroll
  for (int i = 0; i < VPW; ++i) {
    const int byte = (wave + 8 * i) * 1024 + lane * 16;
    const int row = byte / SM::VROW, w = byte % SM::VROW;
    voff[i] = (uint32_t)(row * 64 * 2 + (w < 64 * 2 ? w : 0));
  }
  // K/V tiles go straight to LDS through buffer loads (MUBUF with the lds
  // bit).  The descriptor covers this head's Lp rows exactly (Lp is a
  // multiple of the widest tile, so no tile reaches past it).  The FLAT form
  // of the same DMA would make the compiler wait for every outstanding LDS
  // read (lgkmcnt(0)) while it is in flight.
  const uint32_t head_bytes = (uint32_t)((int64_t)a.Lp * D * 2);
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, head_bytes, kBufferWord3);
  // SelfExtend: grouped keys (at floor(j / G)); coarse / fine: scaled keys
  __amdgpu_buffer_rsrc_t krsrc2 = krsrc;
  if constexpr (MAP != kMapDCA)
    krsrc2 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint16_t*)a.krot2 + bg * (int64_t)a.Lp * D), (short)0, head_bytes, kBufferWord3);
  auto issue_k = [&](int t) {
    const int soff = tile_of(t) * TK * D * 2;
    uint8_t* dst = smem + KB0 + (t & 1) * SM::KBYTES;
    __amdgpu_buffer_rsrc_t rs = krsrc;
    if constexpr (MAP == kMapSelfExtend)
      if (class_of(t) == kSeGrouped) rs = krsrc2;
    if constexpr (MAP == kMapCoarseFine)
      if (t < n_gr) rs = krsrc2;   // the scaled-key pass (same for every wave)
#pragma unroll
    for (int i = 0; i < KPW; ++i)
      if (wave + 8 * i < SM::KPIECES)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (wave + 8 * i) * 1024),
                                                 16, (int)koff[i], soff, 0, 0);
  };
  // V: NSUB consecutive 64-key tiles of the HBM layout.
  auto issue_v = [&](int t) {
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int soff = (tile_of(t) * NSUB + sub) * 64 * D * 2;
      uint8_t* dst = smem + VB0 + (t & 1) * SM::VBYTES + sub * SM::VSUB;
#pragma unroll
      for (int i = 0; i < VPW; ++i)
        if (wave + 8 * i < SM::VPIECES)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (__attribute__((address_space(3))) void*)(dst + (wave + 8 * i) * 1024),
                                                   16, (int)voff[i], soff, 0, 0);
    }
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
  auto do_softmax = [&](int t) {
    const int j0 = tile_of(t) * TK;
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
    auto exps = [&]() {
      float lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g4 = 0; g4 < 4 * NSUB; ++g4) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[g4 >> 1][(g4 & 1) * 8 + e], scale_log2, -m_run));
        const uint4 pu = pack_bf16x8(p);
        float ls = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pu.x), kOnes, lsum[g4 & 3], false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pu.y), kOnes, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pu.z), kOnes, ls, false);
        lsum[g4 & 3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pu.w), kOnes, ls, false);
        pf[g4] = as_bf16x8(pu);
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
  auto prep_q = [&](int t) __attribute__((always_inline)) {
    const int cls = class_of(t);
    if (cls != cur_cls) {
      load_q(cls);
      cur_cls = cls;
    }
  };
  // X(t) for 0 < t < nvt: PV(t-1) then QK(t) as one chain of 32 MFMAs whose
  // LDS operands are read NPRE fragments ahead (a ring of registers), so each
  // MFMA waits only for the oldest read in flight.
  auto x_full = [&](int t) {
    prep_q(t);
    constexpr int NKB = 2 * NSUB;   // 32-key blocks per tile
    constexpr int NPV = 4 * NSUB * NDB, NQK = NKB * NDS, NX = NPV + NQK, NPRE = 6;
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
    }
    // Order: NPRE reads, then (MFMA, read) pairs, then the last MFMAs.
#pragma unroll
    for (int i = 0; i < NPRE; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + NPRE < NX) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  issue_k(0);
  wait_vmem();
  phase_barrier();
  // tile 0 (the first X phase has no PV; the last one, at t = nvt, has no QK)
  if (nvt > 1) issue_k(1);
  issue_v(0);
  if (grp == 0) {
    prep_q(0);
    do_qk(0);
    phase_barrier();
    do_softmax(0);
    wait_vmem();
    phase_barrier();
    for (int t = 1; t < nvt; ++t) {
      if (t + 1 < nvt) issue_k(t + 1);
      issue_v(t);
      x_full(t);
      phase_barrier();
      do_softmax(t);
      wait_vmem();
      phase_barrier();
    }
    do_pv(nvt - 1);
    phase_barrier();
    phase_barrier();
  } else {
    phase_barrier();
    prep_q(0);
    do_qk(0);
    wait_vmem();
    phase_barrier();
    for (int t = 1; t < nvt; ++t) {
      if (t + 1 < nvt) issue_k(t + 1);
      issue_v(t);
      do_softmax(t - 1);
      pin_p();
      phase_barrier();
      x_full(t);
      wait_vmem();
      phase_barrier();
    }
    do_softmax(nvt - 1);
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
        t = a.table[((int64_t)cls * a.L + ii) * HALF + k];
      } else {
        int P;
        if constexpr (MAP == kMapSelfExtend)
          P = cls == kSeNeighbor ? ii : se_query_pos_grouped(ii, a.se_group, W);
        else
          P = query_pos(cls, rqq, s, c);
        t = a.table[(int64_t)P * HALF + k];
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
  // DCA takes the two-group kernel when every 32-row wave block and 64-key
  // tile lies inside one chunk: s a multiple of 64 and query offsets
  // multiples of 32.  SelfExtend always does.  128-key tiles (half the phase
  // barriers per key) whenever the chunk size allows them.
  bool pp = a.s % 64 == 0;
  if (a.per_seq)
    for (int i = 0; i < a.B; ++i) pp = pp && a.seq_q0[i] % 32 == 0;
  if (a.map == kMapCoarseFine && !pp) return hipErrorInvalidValue;   // needs chunk % 64 == 0 (host-checked)
  if (a.map != kMapDCA || pp) {
    const bool wide = a.Lp % 128 == 0 && (a.map == kMapSelfExtend || a.s % 128 == 0);
    const int nqt = (a.q_rows + PP_BR - 1) / PP_BR;
    const dim3 grid((unsigned)((int64_t)nqt * a.B * a.Hq));
    if (a.map == kMapSelfExtend) {
      if (wide) launch_pp<kMapSelfExtend, 2>(a, grid, nqt, xcd_map, scale_log2, st);
      else launch_pp<kMapSelfExtend, 1>(a, grid, nqt, xcd_map, scale_log2, st);
    } else if (a.map == kMapCoarseFine) {
      if (wide) launch_pp<kMapCoarseFine, 2>(a, grid, nqt, xcd_map, scale_log2, st);
      else launch_pp<kMapCoarseFine, 1>(a, grid, nqt, xcd_map, scale_log2, st);
    } else {
      if (wide) launch_pp<kMapDCA, 2>(a, grid, nqt, xcd_map, scale_log2, st);
      else launch_pp<kMapDCA, 1>(a, grid, nqt, xcd_map, scale_log2, st);
    }
    return hipGetLastError();
  }
  const int nqt = (a.q_rows + BR - 1) / BR;
  const dim3 grid((unsigned)((int64_t)nqt * a.B * a.Hq));
  if (a.D == 64)
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, dim3(256), 0, st, a, nqt, xcd_map, scale_log2);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, dim3(256), 0, st, a, nqt, xcd_map, scale_log2);
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
