// decode.hip - DCA decode: one new query token per sequence against a long KV cache.
//
// The new token sits at position q_pos = kv_len - 1, so the result is row
// q_pos of the DCA prefill definition ("Dual-Chunk Attention: Training-Free
// 100k+ Context Guide", sections "The Architecture" .. "Successive Chunk
// Smoothing").  Work is split over the cache ("Strategic Recommendations":
// pair DCA with FlashDecoding, which splits the KV cache across the GPU's
// compute units) and merged by log-sum-exp.
//
// Three launches:
//   1. qprep   : the three rotated variants of every query head (fp64 angles).
//   2. split   : each wave streams one contiguous key range of one (batch,
//                KV head) and keeps an online softmax for the GQA group's query
//                heads (up to 32 per pass, the N side of a 32x32 MFMA).  K and
//                V rows are read with fully coalesced 16-byte loads (with the
//                non-temporal hint: each row is read once) and stored
//                to a per-wave LDS slice as rows (K XOR-swizzled, V padded);
//                the PV operand V^T is read back with the transposing LDS read
//                of gfx950, so no 16-bit scatter stores are needed.  Partials
//                (normalised O and log2-domain LSE) go to the workspace.
//   3. combine : log-sum-exp merge of the partials per query head.
#include "dca_common.hpp"
#include "dca_launch.hpp"

namespace dca {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;
constexpr float kNoMax = -1.0e30f;  // running-max sentinel (finite)
constexpr int SUB = 32;  // keys per wave sub-tile
constexpr int kMaxSplits = 1024;  // partials merged per query head

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

template <int NCK>
__device__ inline int swz(int row, int chunk) {
  if constexpr (NCK == 16)
    return chunk ^ (row & 15);
  else if constexpr (NCK == 8)
    return chunk ^ ((row >> 1) & 7);
  else
    return chunk ^ ((row >> 2) & 3);
}

// ---- 1. query variants -------------------------------------------------------------
// The new token of sequence b sits at (its cached key count) - 1.
__device__ inline int seq_keys(const DecodeArgs& a, int b) { return a.per_seq ? a.seq_len[b] : a.kv_len; }
__host__ __device__ inline int seq_seg(const DecodeArgs& a, int b) { return a.per_seq ? a.seg[b] : 0; }
// Key ranges of sequence b: ceil(keys / kps) ranges of kps keys.  Under the
// two-cache maps a range may hold keys of both caches: keys below seg[b]
// are read from kc2, the others from kc.
__host__ __device__ inline int seq_ranges(int keys, int kps) { return (keys + kps - 1) / kps; }
// Key range `split` of sequence b: [kbeg, kend), empty past its last range.
__device__ inline void range_of(const DecodeArgs& a, int b, int split, int* kbeg, int* kend) {
  const int keys = seq_keys(a, b), kps = a.keys_per_split;
  *kbeg = split * kps;
  *kend = min(*kbeg + kps, keys);
}

template <typename T>
__global__ void decode_qprep_kernel(DecodeArgs a) {
  const int bh = blockIdx.x, k = threadIdx.x;
  const int D = a.D, c = a.c, s = a.s;
  const int half = D / 2;
  if (k >= half) return;
  const T* src = (const T*)a.q + (int64_t)bh * D;
  T* qv = (T*)a.qv;
  const double x1 = Elem<T>::load(src + k), x2 = Elem<T>::load(src + k + half);
  const double theta = pow(a.base, -2.0 * (double)k / (double)D);
  const int qpos = seq_keys(a, bh / a.Hq) - 1;
  const int r = qpos % s;
#pragma unroll
  for (int cls = 0; cls < 3; ++cls) {
    double pos;
    if (a.map == kMapSelfExtend)   // variant 0 grouped, 1 neighbor (2 unused)
      pos = cls == 0 ? (double)se_query_pos_grouped(qpos, a.se_group, a.se_window) : (double)qpos;
    else if (a.map == kMapCoarseFine)
      pos = cf_query_pos(cls, qpos, c, a.cf_inv_kappa);
    else
      pos = (double)query_pos(cls, r, s, c);
    double sn, cs;
    sincos(pos * theta, &sn, &cs);
    T* dst = qv + ((int64_t)bh * 3 + cls) * D;
    Elem<T>::store(dst + k, (float)(x1 * cs - x2 * sn));
    Elem<T>::store(dst + k + half, (float)(x2 * cs + x1 * sn));
  }
}

// ---- 2. split kernel, bf16 MFMA ----------------------------------------------------
// PAGED: the caches are page pools (a.pg); the dense instantiation carries
// none of the block-table work.  TWO: a map with two key caches (SelfExtend,
// coarse / fine); the DCA instantiation carries none of that work.
template <int D, bool PAGED, bool TWO>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_split_bf16_kernel(DecodeArgs a, int nqg, float scale_log2) {
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;             // 16-byte chunks per cache row
  constexpr int NI = SUB * CPR / 64;     // load instructions per sub-tile per tensor
  constexpr int KBYTES = SUB * D * 2;
  // V rows stay row-major in LDS, padded so that both the 16-byte row stores
  // and the transposing fragment reads below are bank-conflict free.
  constexpr int VROWB = D * 2 + 64;
  constexpr int WBYTES = KBYTES + SUB * VROWB;  // K rows + V rows, per wave
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * WBYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, ql = lane & 31;
  // Flat wave index -> (sequence b, key range, unit (KV head g, query group
  // qg)).  Only real ranges get a wave: sequence b has ceil(keys / kps)
  // ranges for each of its Hkv * nqg units.  The unit varies fastest, so the
  // waves of a workgroup (and of neighbouring workgroups) read adjacent
  // head slices of the same cache rows at the same time: whole rows stream
  // out of DRAM together (6 % faster than range-fastest order at the 100k
  // shape, 10 % for a ragged batch).
  const int f = blockIdx.x * 4 + wave;
  const int upq = a.Hkv * nqg;
  int b = 0, rem;
  if (a.per_seq) {
    if (f >= a.wave_start[a.B]) return;
    while (b + 1 < a.B && a.wave_start[b + 1] <= f) ++b;   // wave-uniform scalar loop
    rem = f - a.wave_start[b];
  } else {
    if (f >= a.B * upq * a.nsplit) return;
    b = f / (upq * a.nsplit);
    rem = f - b * upq * a.nsplit;
  }
  const int split = rem / upq;
  const int unit = rem - split * upq;
  const int qg = unit % nqg;
  const int g = unit / nqg;
  const int G = a.Hq / a.Hkv;
  const int qi = qg * 32 + ql;   // index inside the GQA group
  const bool qvalid = qi < G;
  const int hq = g * G + (qvalid ? qi : 0);
  const int kv_len = seq_keys(a, b), s = a.s;
  int kbeg, kend;
  range_of(a, b, split, &kbeg, &kend);
  const int qpos = kv_len - 1;
  const int nq = qpos / s;
  // Two caches: keys below seg come from kc2 (SelfExtend: grouped keys,
  // relation 0; coarse / fine: coarse-scaled keys, relation 2), the others
  // from kc (SelfExtend: neighbor keys, relation 1; coarse / fine: plain keys,
  // relation 0 or 1 by chunk).
  const int seg = TWO ? seq_seg(a, b) : 0;

  uint8_t* kl = smem + wave * WBYTES;
  uint8_t* vl = kl + KBYTES;
  const int64_t row_stride = (int64_t)a.Hkv * D;  // elements between consecutive cache rows
  const uint16_t* kc = (const uint16_t*)a.kc + (int64_t)g * D;
  const uint16_t* kc2 = TWO ? (const uint16_t*)a.kc2 + (int64_t)g * D : kc;
  // cache holding the key rows of the sub-tile starting at j0 (its first key's)
  auto kbase = [&](int j0) { return (TWO && j0 < seg) ? kc2 : kc; };
  const uint16_t* vc = (const uint16_t*)a.vc + (int64_t)g * D;
  const uint16_t* qv = (const uint16_t*)a.qv + ((int64_t)b * a.Hq + hq) * 3 * D;

  bf16x8 qf[NDS];
  auto load_q = [&](int cls) {
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const uint4 u = qvalid ? *(const uint4*)(qv + cls * D + ds * 16 + hh * 8) : make_uint4(0, 0, 0, 0);
      qf[ds] = as_bf16x8(u);
    }
  };

  // Cache rows of keys j0 + 16 h .. j0 + 16 h + 15 (h = 0, 1) are
  // consecutive in both layouts: j0 is a multiple of 32 and a page holds a
  // multiple of 16 rows.  Paged: one (scalar) block-table read per half.
  int64_t rb[2] = {0, 0};
  bool bad = false;   // a block-table entry outside the pool: output NaN
  auto rows_of = [&](int j0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = j0 + 16 * h;
      if constexpr (PAGED) {
        // b and j are wave-uniform, so is the page: keep it in scalar registers
        int page = j < kend ? a.pg.bt[(int64_t)b * a.pg.max_blocks + j / a.pg.page_size] : 0;
        page = __builtin_amdgcn_readfirstlane(page);
        const bool ok = page >= 0 && page < a.pg.num_pages;
        bad |= !ok;
        rb[h] = ok ? (int64_t)page * a.pg.page_size + j % a.pg.page_size : 0;
      } else {
        rb[h] = (int64_t)b * a.cache_len + j;
      }
    }
  };
  // Byte address of a load = (wave-uniform base: the half's first cache row
  // plus the first row of the load instruction) + (one 32-bit lane offset,
  // the same for every load).
  const uint32_t rs2 = (uint32_t)(row_stride * 2);
  const uint32_t lane_off = (uint32_t)(lane / CPR) * rs2 + (uint32_t)(lane % CPR) * 16;
  // lo: lane_off made opaque once per sub-tile, so that the compiler cannot
  // hoist 64-bit per-load addresses out of the key loop (they would not fit
  // in registers next to the accumulators).
  auto paddr = [&](const uint16_t* base, int it, uint32_t lo) __attribute__((always_inline)) {
    const int r0 = it * 64 / CPR;   // first row of load instruction it
    const char* sb = (const char*)(base + rb[r0 >> 4] * row_stride) + (size_t)(r0 & 15) * rs2;
    return (const uint4*)(sb + lo);
  };
  uint4 kreg[NI], vreg[NI];
  auto gload_k = [&](int j0, const uint16_t* kb) {
    uint32_t lo = lane_off;
    asm volatile("" : "+v"(lo));
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int j = j0 + (it * 64 + lane) / CPR;
      kreg[it] = (j < kend) ? load_stream(paddr(kb, it, lo)) : make_uint4(0, 0, 0, 0);
    }
  };
  auto gload_v = [&](int j0) {
    uint32_t lo = lane_off;
    asm volatile("" : "+v"(lo));
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int j = j0 + (it * 64 + lane) / CPR;
      vreg[it] = (j < kend) ? load_stream(paddr(vc, it, lo)) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore_k = [&]() {
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int id = it * 64 + lane;
      const int row = id / CPR, ch = id % CPR;
      *(uint4*)(kl + row * (D * 2) + swz<CPR>(row, ch) * 16) = kreg[it];
    }
  };
  auto lstore_v = [&]() {
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int id = it * 64 + lane;
      const int row = id / CPR, ch = id % CPR;
      *(uint4*)(vl + row * VROWB + ch * 16) = vreg[it];
    }
  };
  // PV operand V^T from row-major V with ds_read_b64_tr_b16: inside each
  // 16-lane group, lane s addresses key row (s / 4) and dims 4*(s % 4)..+3,
  // and the instruction hands lane i four keys at dim i.  Two reads give a
  // lane the 8 keys of its MFMA k-slots: keys hh*4 + 0..3 and 8 + hh*4 + 0..3
  // of the 16-key group (the order the S^T output registers hold P in).
  const int sl = lane & 15;
  const int vtr = (hh * 4 + (sl >> 2)) * VROWB + ((((lane >> 4) & 1) * 16) + (sl & 3) * 4) * 2;
  auto tr_read = [&](const uint8_t* base, int off) -> uint2 {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(base + off));
    return __builtin_bit_cast(uint2, r);
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
  float m_run = kNoMax, l_run = 0.f;
  int cur_cls = -1;

  rows_of(kbeg);
  gload_k(kbeg, kbase(kbeg));
  gload_v(kbeg);
  for (int j0 = kbeg; j0 < kend; j0 += SUB) {
    __builtin_amdgcn_wave_barrier();
    // Store each half as soon as it lands and re-issue it at once, so the
    // other half's loads stay in flight meanwhile.
    const bool more = j0 + SUB < kend;
    lstore_k();
    if (more) {
      rows_of(j0 + SUB);
      gload_k(j0 + SUB, kbase(j0 + SUB));
    }
    lstore_v();
    if (more) gload_v(j0 + SUB);
    __builtin_amdgcn_wave_barrier();

    const int jl = min(j0 + SUB, kend) - 1;
    const bool tail = j0 + SUB > kend;
    // Two caches: a sub-tile holding keys of both is processed twice, first
    // its kc2 keys (staged above), then its kc keys, re-staged from kc.
    const bool two_pass = TWO && j0 < seg && seg <= jl;
    for (int pass = 0; pass < (two_pass ? 2 : 1); ++pass) {
    int plo = j0, phi = jl;   // keys of this pass
    if constexpr (TWO) {
      if (two_pass) {
        if (pass == 0) {
          phi = seg - 1;
        } else {
          plo = seg;
          // K rows of this sub-tile from kc, then the next sub-tile's load
          // again (its registers were taken)
          __builtin_amdgcn_wave_barrier();
          rows_of(j0);
          gload_k(j0, kc);
          lstore_k();
          if (more) {
            rows_of(j0 + SUB);
            gload_k(j0 + SUB, kbase(j0 + SUB));
          }
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
    const bool se = a.map == kMapSelfExtend;
    const int se_cls = (TWO && plo < seg) ? 0 : 1;
    const int cls_lo = se ? se_cls : min(nq - phi / s, 2), cls_hi = se ? se_cls : min(nq - plo / s, 2);
    const bool straddle = cls_lo != cls_hi;
    // A sub-tile spanning several relations is processed once per relation
    // with the other pairs masked; the online softmax merges the pieces.
    for (int cls = cls_lo; cls <= cls_hi; ++cls) {
      if (cls != cur_cls) {
        load_q(cls);
        cur_cls = cls;
      }
      // Keep the fragment reads inside this (rarely repeated) loop.
      int toff = wave * WBYTES;
      asm volatile("" : "+v"(toff));
      const uint8_t* kl = smem + toff;
      const uint8_t* vl = kl + KBYTES;
      const uint8_t* vtb = vl + vtr;
      f32x16 sacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const int ch = ds * 2 + hh;
        const bf16x8 kf = *(const bf16x8*)(kl + ql * (D * 2) + swz<CPR>(ql, ch) * 16);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], sacc, 0, 0, 0);
      }
      if (tail || straddle || two_pass) {
        // Keys kept: the split's range and the pass's keys, intersected on a
        // straddling sub-tile with the key range of relation `cls` (intra:
        // chunk nq, successive: chunk nq-1, inter: chunks < nq-1).
        int lo = max(kbeg, plo), hi = min(kend - 1, phi);
        if (straddle) {
          lo = max(lo, cls == 0 ? nq * s : (cls == 1 ? (nq - 1) * s : 0));
          hi = min(hi, cls == 0 ? qpos : (cls == 1 ? nq * s - 1 : (nq - 1) * s - 1));
        }
        const int jb = j0 + hh * 4;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = jb + (v >> 2) * 8 + (v & 3);
          sacc[v] = (j >= lo && j <= hi) ? sacc[v] : -INFINITY;
        }
      }
      float mx = sacc[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
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
      for (int u = 0; u < 2; ++u) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[u * 8 + e], scale_log2, -m_run));
        // Row sum of the fp32 probabilities (as the prefill kernels sum them).
        lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        const bf16x8 pf = as_bf16x8(pack_bf16x8(p));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint2 lo = tr_read(vtb, u * 16 * VROWB + db * 64);
          const uint2 hi = tr_read(vtb, u * 16 * VROWB + 8 * VROWB + db * 64);
          const bf16x8 vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[db], 0, 0, 0);
        }
      }
      l_run += lsum;
    }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qvalid) {
    const int64_t pidx = ((int64_t)b * a.Hq + hq) * a.nsplit + split;
    float* po = a.part_o + pidx * D;
    // empty range: O 0, LSE -inf; an unreadable page: NaN
    const float inv = (PAGED && bad) ? __builtin_nanf("") : (l_tot > 0.f ? 1.f / l_tot : 0.f);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        float4 o4 = make_float4(oacc[db][grp * 4] * inv, oacc[db][grp * 4 + 1] * inv,
                                oacc[db][grp * 4 + 2] * inv, oacc[db][grp * 4 + 3] * inv);
        *(float4*)(po + db * 32 + grp * 8 + hh * 4) = o4;
      }
    if (hh == 0) a.part_lse[pidx] = (PAGED && bad) ? __builtin_nanf("") : m_run + log2f(l_tot);
  }
}

// ---- 2'. split kernel, fp32 (VALU) -------------------------------------------------
// One workgroup per (batch, query head, split); 256 keys scored per step.
__global__ void __launch_bounds__(256) decode_split_f32_kernel(DecodeArgs a) {
  __shared__ float qs[3][128];
  __shared__ float sc[256];
  __shared__ float red[8];
  const int split = blockIdx.x, bh = blockIdx.y;
  const int D = a.D;
  const int b = bh / a.Hq, hq = bh - b * a.Hq;
  const int G = a.Hq / a.Hkv, g = hq / G;
  const int kv_len = seq_keys(a, b), s = a.s;
  int kbeg, kend;
  range_of(a, b, split, &kbeg, &kend);   // past the sequence's ranges: empty
  const int seg = a.map == kMapDCA ? 0 : seq_seg(a, b);   // keys below seg: from kc2
  const int nq = (kv_len - 1) / s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const float* qv = (const float*)a.qv + (int64_t)bh * 3 * D;
  for (int idx = tid; idx < 3 * D; idx += 256) qs[idx / D][idx % D] = qv[idx];
  const int64_t row_stride = (int64_t)a.Hkv * D;
  const float* kc = (const float*)a.kc + (int64_t)g * D;
  const float* kc2 = a.map == kMapDCA ? kc : (const float*)a.kc2 + (int64_t)g * D;
  const float* vc = (const float*)a.vc + (int64_t)g * D;
  __shared__ int64_t rows[256];   // cache row of each key of the current step (-1: unreadable page)
  float m = -INFINITY, l = 0.f, o = 0.f;  // thread tid < D owns output dim tid
  __syncthreads();
  for (int jb = kbeg; jb < kend; jb += 256) {
    const int j = jb + tid;
    float x = -INFINITY;
    if (j < kend) {
      const int64_t row = cache_row(a.pg, a.cache_len, b, j);
      rows[tid] = row;
      if (row < 0) {
        x = __builtin_nanf("");   // unreadable page: the row's result becomes NaN
      } else {
        const int cls = a.map == kMapSelfExtend ? (j < seg ? 0 : 1) : min(nq - j / s, 2);
        const float* kr = (j < seg ? kc2 : kc) + row * row_stride;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(qs[cls][d], kr[d], acc);
        x = acc * a.sm_scale;
      }
    }
    float mx = x;
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) red[wid] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float mn = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
    const float p = (x == -INFINITY) ? 0.f : expf(x - mn);
    sc[tid] = p;
    float ps = p;
    for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    __syncthreads();
    if (lane == 0) red[4 + wid] = ps;
    __syncthreads();
    l = l * alpha + (red[4] + red[5] + red[6] + red[7]);
    m = mn;
    if (tid < D) {
      float acc = o * alpha;
      const int nk = min(256, kend - jb);
      for (int t = 0; t < nk; ++t)
        acc = fmaf(sc[t], rows[t] < 0 ? 0.f : vc[rows[t] * row_stride + tid], acc);
      o = acc;
    }
    __syncthreads();
  }
  if (tid < D) {
    const int64_t pidx = (int64_t)bh * a.nsplit + split;
    a.part_o[pidx * D + tid] = l > 0.f ? o / l : 0.f;   // empty range: O 0, LSE -inf
    if (tid == 0) a.part_lse[pidx] = (m + logf(l)) * kLog2e;
  }
}

// ---- 3. combine ----------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(128) decode_combine_kernel(DecodeArgs a) {
  // One workgroup per (batch, query head): the split weights 2^(lse_i - M)
  // are computed once into LDS, then every thread sums one output dim.  Only
  // the sequence's own key ranges are merged (ceil(keys / kps) of the nsplit
  // slots).
  __shared__ float wts[kMaxSplits];
  __shared__ float red[2];
  const float* __restrict__ part_o = a.part_o;
  T* __restrict__ o = (T*)a.o;
  float* __restrict__ lse = a.lse;
  const int D = a.D;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int ns = seq_ranges(seq_keys(a, bh / a.Hq), a.keys_per_split);
  const float* pl = a.part_lse + (int64_t)bh * a.nsplit;
  float M = -INFINITY;
  for (int i = tid; i < ns; i += 128) M = fmaxf(M, pl[i]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  float ws = 0.f;
  for (int i = tid; i < ns; i += 128) {
    const float wgt = exp2f(pl[i] - M);
    wts[i] = wgt;
    ws += wgt;
  }
  for (int off = 32; off > 0; off >>= 1) ws += __shfl_xor(ws, off);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = ws;
  __syncthreads();
  const float wsum = red[0] + red[1];
  if (tid < D) {
    const float* po = part_o + (int64_t)bh * a.nsplit * D + tid;
    float acc = 0.f;
    for (int i = 0; i < ns; ++i) acc = fmaf(wts[i], po[(int64_t)i * D], acc);
    Elem<T>::store(o + (int64_t)bh * D + tid, acc / wsum);
  }
  if (tid == 0 && lse) lse[bh] = (M + log2f(wsum)) * kLn2;
}

}  // namespace

void decode_plan(const int64_t* kv, int64_t B, int64_t uniform_kv, int64_t Hq, int64_t Hkv, int dtype,
                 int* keys_per_split, int* nsplit) {
  // One wave per key range, as many ranges as the chip holds at once: MI355X
  // runs 8 of these waves per CU (2 per SIMD) on 256 CUs.  The range length is
  // the shortest multiple of 32 keys whose ranges, over the whole batch (a
  // ragged one too), fit in one such round: one round of long ranges measured
  // faster than several rounds of short ones (fewer prologues, partials and
  // round boundaries), and a second, mostly idle round costs a whole range.
  const int64_t G = Hq / Hkv;
  const int64_t waves_per_key = dtype == 0 ? Hq : Hkv * ((G + 31) / 32);  // waves reading one cached key
  const int64_t target = 2048;
  auto len = [&](int64_t b) { return kv ? kv[b] : uniform_kv; };
  auto ranges = [&](int64_t b, int64_t kps) { return (len(b) + kps - 1) / kps; };
  int64_t max_kv = 0;
  for (int64_t b = 0; b < B; ++b) max_kv = len(b) > max_kv ? len(b) : max_kv;
  auto waves = [&](int64_t kps) {
    if (!kv) return B * ((uniform_kv + kps - 1) / kps) * waves_per_key;
    int64_t n = 0;
    for (int64_t b = 0; b < B; ++b) n += ranges(b, kps);
    return n * waves_per_key;
  };
  // Search in units of SUB keys.  At least 256 keys per range, and at most
  // kMaxSplits ranges per sequence (the combine kernel keeps one weight per
  // range in LDS).  waves() never grows with the range length; if even one
  // range per sequence overflows the round, the whole length is taken.
  const int64_t cap = kMaxSplits;
  int64_t lo = (max_kv + cap - 1) / cap;
  lo = (round_up(lo < 256 ? 256 : lo, SUB)) / SUB;
  int64_t hi = round_up(max_kv, SUB) / SUB;
  if (hi < lo) hi = lo;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (waves(mid * SUB) <= target)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int64_t kps = lo * SUB;
  *keys_per_split = (int)kps;
  int64_t ns = 0;
  for (int64_t b = 0; b < (kv ? B : 1); ++b) ns = ranges(b, kps) > ns ? ranges(b, kps) : ns;
  *nsplit = (int)ns;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t st) {
  const int nbh = a.B * a.Hq;
  if (dtype == 0) {
    hipLaunchKernelGGL(decode_qprep_kernel<float>, dim3(nbh), dim3(64), 0, st, a);
    hipLaunchKernelGGL(decode_split_f32_kernel, dim3(a.nsplit, nbh), dim3(256), 0, st, a);
    hipLaunchKernelGGL(decode_combine_kernel<float>, dim3(nbh), dim3(128), 0, st, a);
  } else {
    hipLaunchKernelGGL(decode_qprep_kernel<uint16_t>, dim3(nbh), dim3(64), 0, st, a);
    const int G = a.Hq / a.Hkv;
    const int nqg = (G + 31) / 32;
    DecodeArgs b = a;
    int64_t waves = (int64_t)a.B * a.Hkv * nqg * a.nsplit;
    if (a.per_seq) {   // flat numbering of the real ranges, sequence by sequence
      b.wave_start[0] = 0;
      for (int i = 0; i < a.B; ++i)
        b.wave_start[i + 1] = b.wave_start[i] + seq_ranges(a.seq_len[i], a.keys_per_split) * a.Hkv * nqg;
      waves = b.wave_start[a.B];
    }
    const dim3 grid((unsigned)((waves + 3) / 4));
    const float scale_log2 = a.sm_scale * kLog2e;
    const bool paged = a.pg.bt != nullptr, two = a.map != kMapDCA;
    if (a.D == 64) {
      if (two && paged)
        hipLaunchKernelGGL((decode_split_bf16_kernel<64, true, true>), grid, dim3(256), 0, st, b, nqg, scale_log2);
      else if (two)
        hipLaunchKernelGGL((decode_split_bf16_kernel<64, false, true>), grid, dim3(256), 0, st, b, nqg, scale_log2);
      else if (paged)
        hipLaunchKernelGGL((decode_split_bf16_kernel<64, true, false>), grid, dim3(256), 0, st, b, nqg, scale_log2);
      else
        hipLaunchKernelGGL((decode_split_bf16_kernel<64, false, false>), grid, dim3(256), 0, st, b, nqg, scale_log2);
    } else {
      if (two && paged)
        hipLaunchKernelGGL((decode_split_bf16_kernel<128, true, true>), grid, dim3(256), 0, st, b, nqg, scale_log2);
      else if (two)
        hipLaunchKernelGGL((decode_split_bf16_kernel<128, false, true>), grid, dim3(256), 0, st, b, nqg, scale_log2);
      else if (paged)
        hipLaunchKernelGGL((decode_split_bf16_kernel<128, true, false>), grid, dim3(256), 0, st, b, nqg, scale_log2);
      else
        hipLaunchKernelGGL((decode_split_bf16_kernel<128, false, false>), grid, dim3(256), 0, st, b, nqg, scale_log2);
    }
    hipLaunchKernelGGL(decode_combine_kernel<uint16_t>, dim3(nbh), dim3(128), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dca
