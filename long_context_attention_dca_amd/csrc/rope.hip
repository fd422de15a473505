// rope.hip - RoPE table, the dca_rope_remap kernel and the prefill K/V prep pass.
//
// RoPE ("Dual-Chunk Attention: Training-Free 100k+ Context Guide", section
// "The Problem"): the pair (x_k, x_{k+D/2}) is turned by position * theta_k,
// theta_k = base^(-2k/D).  DCA positions ("The Architecture" box and the
// intra / inter / successive sections): keys at j mod s, queries at one of
// three positions chosen by the chunk relation.  SelfExtend ("LLM Maybe
// LongLM", abstract) positions: neighbor pairs plain, grouped pairs with keys
// at floor(j / G) and queries at floor(i / G) + W - floor(W / G).
#include "dca_common.hpp"
#include "dca_launch.hpp"

namespace dca {

// ---- cos/sin table (fp64), [npos][D/2] or frequency-major [D/2][npos] -------------------
// Thread idx covers entry idx of the layout it writes, so the stores are
// contiguous either way.
__global__ void rope_table_kernel(double2* __restrict__ table, int npos, int half, int D, double base,
                                  int kmajor) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= npos * half) return;
  int p, k;
  if (kmajor) {
    k = idx / npos;
    p = idx - k * npos;
  } else {
    p = idx / half;
    k = idx - p * half;
  }
  const double theta = pow(base, -2.0 * (double)k / (double)D);
  double sn, cs;
  sincos((double)p * theta, &sn, &cs);
  table[idx] = make_double2(cs, sn);
}

hipError_t launch_rope_table(double2* table, int npos, int D, double base, bool kmajor, hipStream_t st) {
  const int half = D / 2;
  const int n = npos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, table, npos, half, D,
                     base, kmajor ? 1 : 0);
  return hipGetLastError();
}

__global__ void rope_table_f32_kernel(float2* __restrict__ table, int npos, int D, double base) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= npos * (D / 2)) return;
  const int k = idx / npos, p = idx - k * npos;
  const double theta = pow(base, -2.0 * (double)k / (double)D);
  double sn, cs;
  sincos((double)p * theta, &sn, &cs);
  table[idx] = make_float2((float)cs, (float)sn);
}

hipError_t launch_rope_table_f32(float2* table, int npos, int D, double base, hipStream_t st) {
  const int n = npos * (D / 2);
  hipLaunchKernelGGL(rope_table_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, table, npos, D, base);
  return hipGetLastError();
}

__global__ void rope_theta_kernel(double* __restrict__ theta, int half, int D, double base) {
  const int k = threadIdx.x;
  if (k < half) theta[k] = pow(base, -2.0 * (double)k / (double)D);
}

hipError_t launch_rope_theta(double* theta, int D, double base, hipStream_t st) {
  hipLaunchKernelGGL(rope_theta_kernel, dim3(1), dim3(64), 0, st, theta, D / 2, D, base);
  return hipGetLastError();
}

// Frequency-major: entry (cls * L + i, k) at k * 3L + cls * L + i; fp64 or
// rounded to fp32.
__device__ inline void put_cs(double2* p, double2 v) { *p = v; }
__device__ inline void put_cs(float2* p, double2 v) { *p = make_float2((float)v.x, (float)v.y); }

template <typename T>
__global__ void cf_query_table_kernel(T* __restrict__ tab, int L, int C, double inv_kappa,
                                      const double* __restrict__ theta) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x, cls = blockIdx.y, k = blockIdx.z;
  if (i < L)
    put_cs(tab + (int64_t)k * 3 * L + (int64_t)cls * L + i, rope_cs(cf_query_pos(cls, i, C, inv_kappa), theta[k]));
}

template <typename T>
static hipError_t cf_query_table(T* tab, int L, int D, int C, double inv_kappa, const double* theta,
                                 hipStream_t st) {
  hipLaunchKernelGGL(cf_query_table_kernel<T>, dim3((L + 255) / 256, 3, D / 2), dim3(256), 0, st, tab, L, C,
                     inv_kappa, theta);
  return hipGetLastError();
}

hipError_t launch_cf_query_table(double2* tab, int L, int D, int C, double inv_kappa, const double* theta,
                                 hipStream_t st) {
  return cf_query_table(tab, L, D, C, inv_kappa, theta, st);
}

hipError_t launch_cf_query_table_f32(float2* tab, int L, int D, int C, double inv_kappa, const double* theta,
                                     hipStream_t st) {
  return cf_query_table(tab, L, D, C, inv_kappa, theta, st);
}

// ---- dca_rope_remap -----------------------------------------------------------------
// One workgroup per kRemapTokens consecutive tokens: the angles of their
// positions are made once in fp64 (one (token, k) pair per thread) and applied
// to every (batch, head) row of those tokens, 16 bytes per load and store.
// Maps 0-4 take the DCA (c, w); the SelfExtend maps 5 and 6 take c = G and
// w = W.
__device__ inline int64_t remap_position(int64_t p, int map, int c, int w) {
  const int64_t s = c - w;
  switch (map) {
    case 5:  // SelfExtend grouped key
      return p / c;
    case 6:  // SelfExtend grouped query
      return p / c + w - w / c;
    case 0:  // key
    case 1:  // query, intra
      return p % s;
    case 2: {  // query, successive
      const int64_t r = p % s;
      return (s + r < c) ? s + r : (int64_t)(c - 1);
    }
    case 3:  // query, inter
      return c - 1;
    default:  // plain RoPE
      return p;
  }
}

// 16 bytes of T: 8 bf16 or 4 fp32 values, widened to float.
template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& u, float* f) { unpack_bf16x8(u, f); }
  __device__ static uint4 pack(const float* f) { return pack_bf16x8(f); }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

// fp64 -> fp32 rounded to odd (round to nearest, then the odd neighbour when
// that was inexact).  The 16 bits fp32 holds beyond bf16 keep the later
// rounding to bf16 exact, so fp64 -> bf16 is rounded once, to nearest even,
// whatever the compiler makes of the two conversions.
__device__ inline float f32_round_odd(double d) {
  const float f = (float)d;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != d && (u & 1u) == 0) u += fabs(d) > fabs(back) ? 1u : 0xffffffffu;
  return __uint_as_float(u);
}

// Turn the pairs (x1[e], x2[e]) by the angles cs[e] = (cos, sin): fp64
// arithmetic with the fma written out, so every caller computes the same
// fp64 values, then the value handed back for T's single rounding.
template <typename T, int N>
__device__ inline void rotate_pairs(float* x1, float* x2, const double2* cs) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const double a = x1[e], b = x2[e];
    const double y1 = fma(a, cs[e].x, -(b * cs[e].y));
    const double y2 = fma(b, cs[e].x, a * cs[e].y);
    if constexpr (sizeof(T) == 2) {
      x1[e] = f32_round_odd(y1);
      x2[e] = f32_round_odd(y2);
    } else {
      x1[e] = (float)y1;
      x2[e] = (float)y2;
    }
  }
}

constexpr int kRemapTokens = 4;

template <typename T, int D>
__global__ void __launch_bounds__(256) rope_remap_kernel(const T* __restrict__ x, T* __restrict__ out,
                                                         int64_t B, int64_t L, int H, int64_t pos0, int map,
                                                         int c, int w, double base, double step) {
  constexpr int half = D / 2, N = Vec16<T>::N, NG = half / N;   // 16-byte groups per half row
  __shared__ double2 cs[kRemapTokens][half];
  const int64_t t0 = (int64_t)blockIdx.x * kRemapTokens;
  const int ntok = (int)(L - t0 < kRemapTokens ? L - t0 : kRemapTokens);
  for (int idx = threadIdx.x; idx < ntok * half; idx += 256) {
    const int tk = idx / half, k = idx - tk * half;
    const int64_t p = pos0 + t0 + tk;
    const double P = map == kRemapCoarseScaled ? (double)(p / c) * step + (double)(p % c)
                                               : (double)remap_position(p, map, c, w);
    const double theta = pow(base, -2.0 * (double)k / (double)D);
    double sn, cn;
    sincos(P * theta, &sn, &cn);
    cs[tk][k] = make_double2(cn, sn);
  }
  __syncthreads();
  // Items (b, token, head, group) with the group fastest: a sequence's rows of
  // these tokens are one contiguous run.  The batch index advances by
  // subtraction, so no 64-bit division is made per item.
  const int inner = ntok * H * NG;
  int64_t b = threadIdx.x / inner;
  int r = threadIdx.x - (int)b * inner;
  const int step_b = 256 / inner, step_r = 256 - step_b * inner;
  for (; b < B;) {
    const int g = r % NG, th = r / NG, h = th % H, tk = th / H;
    const int64_t off = ((b * L + t0 + tk) * H + h) * D + g * N;
    float x1[N], x2[N];
    Vec16<T>::unpack(load_stream((const uint4*)(x + off)), x1);
    Vec16<T>::unpack(load_stream((const uint4*)(x + off + half)), x2);
    rotate_pairs<T, N>(x1, x2, &cs[tk][g * N]);
    store_stream((uint4*)(out + off), Vec16<T>::pack(x1));
    store_stream((uint4*)(out + off + half), Vec16<T>::pack(x2));
    b += step_b;
    r += step_r;
    if (r >= inner) {
      r -= inner;
      ++b;
    }
  }
}

template <typename T>
static void launch_remap_t(const void* x, void* out, int64_t B, int64_t L, int64_t H, int64_t D, int64_t pos0,
                           int map, int c, int w, double base, hipStream_t st, double step) {
  const dim3 grid((unsigned)((L + kRemapTokens - 1) / kRemapTokens));
  if (D == 64)
    hipLaunchKernelGGL((rope_remap_kernel<T, 64>), grid, dim3(256), 0, st, (const T*)x, (T*)out, B, L, (int)H,
                       pos0, map, c, w, base, step);
  else
    hipLaunchKernelGGL((rope_remap_kernel<T, 128>), grid, dim3(256), 0, st, (const T*)x, (T*)out, B, L, (int)H,
                       pos0, map, c, w, base, step);
}

hipError_t launch_rope_remap(const void* x, void* out, int64_t B, int64_t L, int64_t H, int64_t D,
                             int64_t pos0, int map, int c, int w, double base, int dtype,
                             hipStream_t st, double step) {
  if (L == 0 || B == 0 || H == 0) return hipSuccess;
  if (dtype == 0)
    launch_remap_t<float>(x, out, B, L, H, D, pos0, map, c, w, base, st, step);
  else
    launch_remap_t<uint16_t>(x, out, B, L, H, D, pos0, map, c, w, base, st, step);
  return hipGetLastError();
}

// ---- prefill K/V prep ---------------------------------------------------------------
// Within each 16-key group of a V^T tile the keys are stored in the order
// 0-3, 8-11, 4-7, 12-15 (bits 2 and 3 of the key index swapped).  That is the
// order in which one half-wave holds the probabilities of a 16-key step in the
// 32x32 MFMA output layout, so the PV step reads 8 contiguous keys per lane.
__device__ inline int vt_perm(int p) { return (p & ~15) | (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1); }

// fp32 prepare pass (keys only; the fp32 kernels read V as it is): one
// workgroup per (64-key tile, KV head, sequence), one rotary pair per thread.
template <int D>
__global__ void __launch_bounds__(256) kv_prep_f32_kernel(KvPrepArgs a) {
  constexpr int half = D / 2;
  constexpr int TK = kPrefillTileKeys;
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int j0 = tile * TK;
  const int Lb = a.per_seq ? a.seq_len[b] : a.L;   // valid rows of this sequence
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const float* k = (const float*)a.k;
  float* krot = (float*)a.krot;
  float* k_rot_out = (float*)a.k_rot_out;
  for (int idx = threadIdx.x; idx < TK * half; idx += 256) {
    const int row = idx / half, kk = idx - row * half;
    const int j = j0 + row;
    float* dst = krot + (bg * a.Lp + j) * D + kk;
    const int64_t crow = j < Lb ? cache_row(a.pg, a.in_rows, b, j) : 0;
    float y1 = 0.f, y2 = 0.f;   // rows past the sequence: zero
    if (j < Lb && crow < 0) {   // unreadable page: poison the key so the rows using it give NaN
      y1 = y2 = __builtin_nanf("");
    } else if (j < Lb) {
      const int64_t in = (crow * a.Hkv + g) * D + kk;
      const double x1 = k[in], x2 = k[in + half];
      if (a.table || a.pos_mode == 1) {
        const double2 c = a.pos_mode == 1
                              ? rope_cs((double)(j / a.cf_chunk) * a.cf_step + (double)(j % a.cf_chunk),
                                        a.theta[kk])
                              : a.table[((j / a.kdiv) % a.kmod) * half + kk];
        y1 = (float)fma(x1, c.x, -(x2 * c.y));   // as rotate_pairs<float>
        y2 = (float)fma(x2, c.x, x1 * c.y);
        if (k_rot_out) {
          k_rot_out[in] = y1;
          k_rot_out[in + half] = y2;
        }
      } else {   // already rotated: exact copy
        y1 = (float)x1;
        y2 = (float)x2;
      }
    }
    dst[0] = y1;
    dst[half] = y2;
  }
}

// bf16 prepare pass with 16-byte accesses throughout.  One workgroup per
// (64-key tile, group of up to kPrepHeads KV heads, sequence).  A thread owns
// (key row, 8-dim group) items: it gets the item's cos/sin once and applies
// them to every head of the group.  The V rows of all the group's heads are
// loaded before the key work, so their loads are in flight meanwhile, then
// each head's tile is transposed through LDS and written as whole 16-byte
// runs of 8 keys (in the key order of vt_perm).
constexpr int kPrepHeads = 2;

template <int D>
__global__ void __launch_bounds__(256) kv_prep_bf16_kernel(KvPrepArgs a) {
  constexpr int half = D / 2, NG = half / 8;             // 8-dim groups per half row
  constexpr int TK = kPrefillTileKeys;
  constexpr int KITEMS = TK * NG / 256;                  // key items per thread
  constexpr int VG = D / 8;                              // 8-dim groups per V row
  constexpr int VITEMS = TK * VG / 256;                  // V loads per thread and head
  constexpr int OITEMS = D * (TK / 8) / 256;             // V^T stores per thread and head
  static_assert(KITEMS >= 1 && VITEMS >= 1 && OITEMS >= 1, "tile too small for the workgroup");
  const int tile = blockIdx.x, b = blockIdx.z, h0 = blockIdx.y * kPrepHeads;
  const int nh = a.Hkv - h0 < kPrepHeads ? a.Hkv - h0 : kPrepHeads;
  const int j0 = tile * TK;
  const int Lb = a.per_seq ? a.seq_len[b] : a.L;   // valid rows of this sequence
  const uint16_t* k = (const uint16_t*)a.k;
  const uint16_t* vv = (const uint16_t*)a.v;
  const bool with_v = a.vt != nullptr;
  const bool rotate = a.table != nullptr || a.pos_mode != 0;
  // pos_mode 2: theta_k once per workgroup, as the table kernel makes it
  __shared__ double theta_s[half];
  if (a.pos_mode == 2) {
    if (threadIdx.x < half) theta_s[threadIdx.x] = pow(a.base, -2.0 * (double)threadIdx.x / (double)D);
    __syncthreads();
  }

  // V rows of every head of the group (zero past the valid rows and for
  // unreadable pages).
  uint4 vr[kPrepHeads][VITEMS];
  if (with_v) {
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int item = threadIdx.x + it * 256;
      const int row = item / VG, dg = item - row * VG;
      const int j = j0 + row;
      const int64_t crow = j < Lb ? cache_row(a.pg, a.in_rows, b, j) : -1;
#pragma unroll
      for (int hh = 0; hh < kPrepHeads; ++hh)
        vr[hh][it] = (hh < nh && crow >= 0) ? load_stream((const uint4*)(vv + (crow * a.Hkv + h0 + hh) * D + dg * 8))
                                            : make_uint4(0, 0, 0, 0);
    }
  }

  // Keys.
#pragma unroll
  for (int it = 0; it < KITEMS; ++it) {
    const int item = threadIdx.x + it * 256;
    const int row = item / NG, kg = item - row * NG;
    const int j = j0 + row, k0 = kg * 8;
    const int64_t crow = j < Lb ? cache_row(a.pg, a.in_rows, b, j) : 0;
    const bool valid = j < Lb && crow >= 0;
    uint4 x1[kPrepHeads], x2[kPrepHeads];
#pragma unroll
    for (int hh = 0; hh < kPrepHeads; ++hh)
      if (hh < nh && valid) {
        const uint16_t* src = k + (crow * a.Hkv + h0 + hh) * D + k0;
        x1[hh] = load_stream((const uint4*)src);
        x2[hh] = load_stream((const uint4*)(src + half));
      }
    double2 cs[8];
    if (valid && rotate) {
      if (a.pos_mode == 1) {
        const double pos = (double)(j / a.cf_chunk) * a.cf_step + (double)(j % a.cf_chunk);
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] = rope_cs(pos, a.theta[k0 + e]);
      } else if (a.pos_mode == 2) {
        const double pos = (double)((j / a.kdiv) % a.kmod);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          double sn, cn;
          sincos(pos * theta_s[k0 + e], &sn, &cn);
          cs[e] = make_double2(cn, sn);
        }
      } else {
        const double2* t = a.table + (int64_t)((j / a.kdiv) % a.kmod) * half + k0;
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] = t[e];
      }
    }
    const uint32_t nan2 = 0x7fc07fc0u;   // two bf16 quiet NaNs
#pragma unroll
    for (int hh = 0; hh < kPrepHeads; ++hh) {
      if (hh >= nh) continue;
      uint16_t* dst = (uint16_t*)a.krot + (((int64_t)b * a.Hkv + h0 + hh) * a.Lp + j) * D + k0;
      uint4 y1, y2;
      if (j >= Lb) {
        y1 = y2 = make_uint4(0, 0, 0, 0);
      } else if (crow < 0) {   // unreadable page: poison the key so the rows using it give NaN
        y1 = y2 = make_uint4(nan2, nan2, nan2, nan2);
      } else if (rotate) {
        float f1[8], f2[8];
        unpack_bf16x8(x1[hh], f1);
        unpack_bf16x8(x2[hh], f2);
        rotate_pairs<uint16_t, 8>(f1, f2, cs);
        y1 = pack_bf16x8(f1);
        y2 = pack_bf16x8(f2);
        if (a.k_rot_out) {
          uint16_t* ko = (uint16_t*)a.k_rot_out + (crow * a.Hkv + h0 + hh) * D + k0;
          *(uint4*)ko = y1;
          *(uint4*)(ko + half) = y2;
        }
      } else {   // already rotated: exact copy
        y1 = x1[hh];
        y2 = x2[hh];
      }
      *(uint4*)dst = y1;
      *(uint4*)(dst + half) = y2;
    }
  }

  // pos_mode 2: this launch also writes the cos / sin table of positions
  // 0 .. table_rows - 1 in fp32, frequency-major ([D/2][table_rows]), a slice
  // per workgroup.
  if (a.pos_mode == 2 && a.table_out) {
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
    const int64_t wg = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t n = (int64_t)a.table_rows * half;
    for (int64_t idx = wg * 256 + threadIdx.x; idx < n; idx += nwg * 256) {
      const int kk = (int)(idx / a.table_rows), p = (int)(idx - (int64_t)kk * a.table_rows);
      double sn, cn;
      sincos((double)p * theta_s[kk], &sn, &cn);
      a.table_out[idx] = make_float2((float)cn, (float)sn);
    }
  }

  // V^T tiles, one head at a time through LDS.
  if (!with_v) return;
  __shared__ __attribute__((aligned(16))) uint16_t vs[TK][D + 8];
  const int ntiles = a.Lp / TK;
  for (int hh = 0; hh < nh; ++hh) {
    if (hh > 0) __syncthreads();   // the previous head's reads are done
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int item = threadIdx.x + it * 256;
      const int row = item / VG, dg = item - row * VG;
      uint4 u = vr[0][it];
#pragma unroll
      for (int x = 1; x < kPrepHeads; ++x)
        if (x == hh) u = vr[x][it];
      *(uint4*)&vs[row][dg * 8] = u;
    }
    __syncthreads();
    uint16_t* dst = (uint16_t*)a.vt + ((((int64_t)b * a.Hkv + h0 + hh) * ntiles + tile) * D) * TK;
#pragma unroll
    for (int it = 0; it < OITEMS; ++it) {
      const int item = threadIdx.x + it * 256;
      const int d = item / (TK / 8), kg = item - d * (TK / 8);
      uint16_t e[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) e[x] = vs[vt_perm(kg * 8 + x)][d];
      *(uint4*)(dst + d * TK + kg * 8) =
          make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16), e[4] | ((uint32_t)e[5] << 16),
                     e[6] | ((uint32_t)e[7] << 16));
    }
  }
}

hipError_t launch_kv_prep(const KvPrepArgs& a, int dtype, hipStream_t st) {
  if (dtype == 0) {
    const dim3 grid((unsigned)(a.Lp / kPrefillTileKeys), (unsigned)a.Hkv, (unsigned)a.B);
    if (a.D == 64)
      hipLaunchKernelGGL((kv_prep_f32_kernel<64>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((kv_prep_f32_kernel<128>), grid, dim3(256), 0, st, a);
  } else {
    const dim3 grid((unsigned)(a.Lp / kPrefillTileKeys), (unsigned)((a.Hkv + kPrepHeads - 1) / kPrepHeads),
                    (unsigned)a.B);
    if (a.D == 64)
      hipLaunchKernelGGL((kv_prep_bf16_kernel<64>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((kv_prep_bf16_kernel<128>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dca
