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

#include <mutex>

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

// The bf16 form of rotate_pairs on packed bf16 words (2 values each), with
// the same results and fewer operations.  The fp64 value y goes to fp32
// (round to nearest even) and then to bf16.  The two roundings equal the
// single one except when the fp32 value is itself a midpoint between two bf16
// numbers (low 16 bits 0x8000) without being y: a value on either side of a
// bf16 midpoint cannot cross it when rounded to fp32, since the midpoint is an
// fp32 number.  Where any active lane of the wave meets that case (about one
// value in 65536), the whole wave redoes its pairs through rotate_pairs'
// round-to-odd step instead.
template <int W>
__device__ inline void rotate_bf16_words(const uint32_t* w1, const uint32_t* w2, const double2* cs, uint32_t* o1,
                                         uint32_t* o2) {
  constexpr int N = 2 * W;
  float f1[N], f2[N];
  uint64_t midpoint = 0;   // lanes with an fp32 value on a bf16 midpoint (one compare per value)
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const double a = __uint_as_float(e & 1 ? w1[e / 2] & 0xffff0000u : w1[e / 2] << 16);
    const double b = __uint_as_float(e & 1 ? w2[e / 2] & 0xffff0000u : w2[e / 2] << 16);
    f1[e] = (float)fma(a, cs[e].x, -(b * cs[e].y));
    f2[e] = (float)fma(b, cs[e].x, a * cs[e].y);
    midpoint |= __builtin_amdgcn_ballot_w64((__float_as_uint(f1[e]) & 0xffffu) == 0x8000u);
    midpoint |= __builtin_amdgcn_ballot_w64((__float_as_uint(f2[e]) & 0xffffu) == 0x8000u);
  }
  if (midpoint != 0) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      f1[e] = __uint_as_float(e & 1 ? w1[e / 2] & 0xffff0000u : w1[e / 2] << 16);
      f2[e] = __uint_as_float(e & 1 ? w2[e / 2] & 0xffff0000u : w2[e / 2] << 16);
    }
    rotate_pairs<uint16_t, N>(f1, f2, cs);
  }
#pragma unroll
  for (int q = 0; q < W; ++q) {
    o1[q] = pack_bf16x2(f1[2 * q], f1[2 * q + 1]);
    o2[q] = pack_bf16x2(f2[2 * q], f2[2 * q + 1]);
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
    const uint4 u1 = load_stream((const uint4*)(x + off)), u2 = load_stream((const uint4*)(x + off + half));
    if constexpr (sizeof(T) == 2) {
      const uint32_t w1[4] = {u1.x, u1.y, u1.z, u1.w}, w2[4] = {u2.x, u2.y, u2.z, u2.w};
      uint32_t o1[4], o2[4];
      rotate_bf16_words<4>(w1, w2, &cs[tk][g * N], o1, o2);
      store_stream((uint4*)(out + off), make_uint4(o1[0], o1[1], o1[2], o1[3]));
      store_stream((uint4*)(out + off + half), make_uint4(o2[0], o2[1], o2[2], o2[3]));
    } else {
      float x1[N], x2[N];
      Vec16<T>::unpack(u1, x1);
      Vec16<T>::unpack(u2, x2);
      rotate_pairs<T, N>(x1, x2, &cs[tk][g * N]);
      store_stream((uint4*)(out + off), Vec16<T>::pack(x1));
      store_stream((uint4*)(out + off + half), Vec16<T>::pack(x2));
    }
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

// bf16 prepare pass.  Every wave works through its own share of a flat list of
// units in which K and V units are interleaved in proportion, so that the
// reads, the writes and the K rotation's fp64 arithmetic of different waves
// overlap; past the workgroup's start (where the first wave makes the
// frequencies theta_k into LDS) no wave waits for another.
//  * K unit: RK consecutive key rows (RK = 256 / D: 2 for D 128, 4 for
//    D 64) of one sequence and up to kPrepKeyHeads KV heads.  A lane owns one
//    row and 2 frequencies: it makes their cos/sin pairs once and turns those
//    pairs in every head of the unit (4-byte loads and stores; 32 lanes cover
//    a half row, one 128-byte run).
//  * V unit: 64 keys x 64 dims of one head.  In two halves of 32 keys, the
//    wave writes the rows into its own LDS rows transposed (one LDS row per
//    dim, keys in the order of vt_perm), then stores each dim's keys as
//    16-byte runs of 8; the two halves of every 128-byte V^T line come from
//    the same wave moments apart.
// The grid is twice the workgroups that fit on the chip at once; wave w takes
// units w, w + W, w + 2W, ... (W waves in all).
constexpr int kPrepKeyHeads = 8;
constexpr int kPrepKeyWords = 1;   // 32-bit words (2 frequencies each) per lane and half row
constexpr int kPrepVKeys = 64;     // keys per V unit
constexpr int kPrepVRow = kPrepVKeys / 2 + 8;   // LDS row of one dim, half a V unit's keys, bf16

// NW consecutive 32-bit words with the non-temporal hint / a plain store.
template <int NW>
__device__ inline void load_words(const uint16_t* p, uint32_t* w) {
  if constexpr (NW == 1) {
    w[0] = __builtin_nontemporal_load((const uint32_t*)p);
  } else {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 t = __builtin_nontemporal_load((const u32x2*)p);
    w[0] = t[0];
    w[1] = t[1];
  }
}
template <int NW>
__device__ inline void store_words(uint16_t* p, const uint32_t* w) {
  if constexpr (NW == 1)
    *(uint32_t*)p = w[0];
  else
    *(uint2*)p = make_uint2(w[0], w[1]);
}
// LDS written by some lanes of this wave, then read by others.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// PM: 0 = copy (keys already rotated), 1 = real positions from a.theta
// (pos_mode 1), 2 = cos/sin made here from a.base (pos_mode 2).
template <int D, int PM, bool PAGED>
__global__ void __launch_bounds__(256) kv_prep_bf16_kernel(KvPrepArgs a, int64_t nK, int64_t nV) {
  constexpr int half = D / 2, NW = kPrepKeyWords, NF = 2 * NW, NKG = half / NF, RK = 64 / NKG, ND = D / 64;
  constexpr int KH = kPrepKeyHeads;
  constexpr bool rotate = PM != 0;
  __shared__ double theta_s[half];
  __shared__ __attribute__((aligned(16))) uint16_t vsh[4][64][kPrepVRow];
  if (PM == 2) {
    if (threadIdx.x < half) theta_s[threadIdx.x] = pow(a.base, -2.0 * (double)threadIdx.x / (double)D);
    __syncthreads();
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t W = (int64_t)gridDim.x * 4, N = nK + nV;
  const uint16_t* kin = (const uint16_t*)a.k;
  const uint16_t* vin = (const uint16_t*)a.v;
  const int nRG = a.Lp / RK, nHG = (a.Hkv + KH - 1) / KH, nT = a.Lp / kPrefillTileKeys;
  const int64_t rowstride = (int64_t)a.Hkv * D;   // elements per input row
  for (int64_t u = (int64_t)blockIdx.x * 4 + wave; u < N; u += W) {
    // the lane index is re-read per unit so that the compiler does not keep
    // both unit kinds' lane offsets in registers across the loop
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int64_t kc = u * nK / N;   // K units before unit u
    if ((u + 1) * nK / N > kc) {
      // ---- K unit kc: (sequence b, row group g, head group hg)
      const int hg = (int)(kc % nHG);
      const int64_t bg = kc / nHG;
      const int g = (int)(bg % nRG), b = (int)(bg / nRG);
      const int r = lane / NKG, k0 = (lane % NKG) * NF;
      const int j = g * RK + r;
      const int Lb = a.per_seq ? a.seq_len[b] : a.L;   // valid rows of this sequence
      const int h0 = hg * KH, nh = a.Hkv - h0 < KH ? a.Hkv - h0 : KH;
      const int64_t crow = PAGED ? (j < Lb ? cache_row(a.pg, a.in_rows, b, j) : 0) : (int64_t)b * a.in_rows + j;
      const bool valid = j < Lb && crow >= 0;
      double2 cs[NF];
      if (rotate && valid) {
        if (PM == 1) {
          const double pos = (double)(j / a.cf_chunk) * a.cf_step + (double)(j % a.cf_chunk);
#pragma unroll
          for (int e = 0; e < NF; ++e) cs[e] = rope_cs(pos, a.theta[k0 + e]);
        } else {
          const double pos = (double)((j / a.kdiv) % a.kmod);
#pragma unroll
          for (int e = 0; e < NF; ++e) {
            double sn, cn;
            sincos(pos * theta_s[k0 + e], &sn, &cn);
            cs[e] = make_double2(cn, sn);
          }
        }
      }
      // the angles first, then the loads: their registers are not live together
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* src;
      if (PAGED) {
        src = kin + (crow * a.Hkv + h0) * D + k0;
      } else {   // wave-uniform base + 32-bit lane offset
        const uint16_t* base = kin + ((int64_t)b * a.in_rows + (int64_t)g * RK) * rowstride + h0 * D;
        src = base + (uint32_t)(r * rowstride + k0);
      }
      uint32_t x1[KH][NW], x2[KH][NW];
#pragma unroll
      for (int hh = 0; hh < KH; ++hh)
        if (hh < nh && valid) {
          load_words<NW>(src + hh * D, x1[hh]);
          load_words<NW>(src + hh * D + half, x2[hh]);
        }
      uint16_t* dst = (uint16_t*)a.krot + (((int64_t)b * a.Hkv + h0) * a.Lp + (int64_t)g * RK) * D + r * D + k0;
      const uint32_t nan2 = 0x7fc07fc0u;   // two bf16 quiet NaNs
#pragma unroll
      for (int hh = 0; hh < KH; ++hh) {
        if (hh >= nh) continue;
        uint32_t y1[NW], y2[NW];
        if (j >= Lb) {
#pragma unroll
          for (int q = 0; q < NW; ++q) y1[q] = y2[q] = 0;
        } else if (!valid) {   // unreadable page: poison the key so the rows using it give NaN
#pragma unroll
          for (int q = 0; q < NW; ++q) y1[q] = y2[q] = nan2;
        } else if (rotate) {
          rotate_bf16_words<NW>(x1[hh], x2[hh], cs, y1, y2);
          if (a.k_rot_out) {
            uint16_t* ko = (uint16_t*)a.k_rot_out + (crow * a.Hkv + h0 + hh) * D + k0;
            store_words<NW>(ko, y1);
            store_words<NW>(ko + half, y2);
          }
        } else {   // already rotated: exact copy
#pragma unroll
          for (int q = 0; q < NW; ++q) {
            y1[q] = x1[hh][q];
            y2[q] = x2[hh][q];
          }
        }
        uint16_t* d = dst + (int64_t)hh * a.Lp * D;
        store_words<NW>(d, y1);
        store_words<NW>(d + half, y2);
      }
    } else {
      // ---- V unit u - kc: (sequence b, 64-key tile t, head h, dims dh * 64 ..)
      constexpr int VL = kPrepVKeys / 8;   // 16-byte loads per lane
      int64_t vv = u - kc;
      const int dh = (int)(vv % ND);
      vv /= ND;
      const int h = (int)(vv % a.Hkv);
      vv /= a.Hkv;
      const int t = (int)(vv % nT), b = (int)(vv / nT);
      const int Lb = a.per_seq ? a.seq_len[b] : a.L;
      const int jb = t * kPrefillTileKeys;
      // zero past the valid rows and for unreadable pages; lane item it holds
      // 8 dims of key row (lane >> 3) + 8 * it
      uint4 x[VL];
#pragma unroll
      for (int it = 0; it < VL; ++it) {
        const int i = lane + it * 64, row = i >> 3, dg = i & 7;
        const int j = jb + row;
        if (PAGED) {
          const int64_t crow = j < Lb ? cache_row(a.pg, a.in_rows, b, j) : -1;
          x[it] = crow >= 0 ? load_stream((const uint4*)(vin + (crow * a.Hkv + h) * D + dh * 64 + dg * 8))
                            : make_uint4(0, 0, 0, 0);
        } else {
          const uint16_t* base = vin + ((int64_t)b * a.in_rows + jb) * rowstride + h * D + dh * 64;
          x[it] = j < Lb ? load_stream((const uint4*)(base + (uint32_t)(row * rowstride + dg * 8)))
                         : make_uint4(0, 0, 0, 0);
        }
      }
      // transposed in two halves of 32 keys through the wave's 32-key LDS rows
      // (vt_perm keeps each 16-key group in place, so a half is self-contained)
      uint16_t(*vs)[kPrepVRow] = vsh[wave];
      uint16_t* dst = (uint16_t*)a.vt + ((((int64_t)b * a.Hkv + h) * nT + t) * D + dh * 64) * kPrefillTileKeys;
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        if (hk) wave_lds_sync();   // the first half's LDS reads come before these writes
#pragma unroll
        for (int it = hk * VL / 2; it < (hk + 1) * VL / 2; ++it) {
          const int i = lane + it * 64, row = (i >> 3) - hk * 32, dg = i & 7;
          const int slot = vt_perm(row);
          const uint32_t w4[4] = {x[it].x, x[it].y, x[it].z, x[it].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            vs[dg * 8 + 2 * q][slot] = (uint16_t)(w4[q] & 0xffffu);
            vs[dg * 8 + 2 * q + 1][slot] = (uint16_t)(w4[q] >> 16);
          }
        }
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int i = lane + it * 64, dl = i >> 2, kg = i & 3;
          *(uint4*)(dst + dl * kPrefillTileKeys + hk * 32 + kg * 8) = *(const uint4*)&vs[dl][kg * 8];
        }
      }
      wave_lds_sync();   // this unit's LDS reads come before the next unit's writes
    }
  }

  // PM 2: this launch also writes the cos / sin table of positions
  // 0 .. table_rows - 1 in fp32, frequency-major ([D/2][table_rows]), a slice
  // per wave.
  if (PM == 2 && a.table_out) {
    const int n = a.table_rows * half;
    for (int64_t idx = ((int64_t)blockIdx.x * 4 + wave) * 64 + (threadIdx.x & 63); idx < n; idx += W * 64) {
      const int kk = (int)(idx / a.table_rows), p = (int)(idx - (int64_t)kk * a.table_rows);
      double sn, cn;
      sincos((double)p * theta_s[kk], &sn, &cn);
      a.table_out[idx] = make_float2((float)cn, (float)sn);
    }
  }
}

// Workgroups of a kernel that fit on the current device at once (cached per
// device and kernel).
constexpr int kMaxPrepDevices = 64;
std::mutex g_prep_grid_mutex;

template <typename K>
static hipError_t resident_workgroups(K kernel, int* out) {
  static int cache[kMaxPrepDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxPrepDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_prep_grid_mutex);
  if (cache[dev] == 0) {
    int per_cu = 0, ncu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cache[dev] = per_cu * ncu > 0 ? per_cu * ncu : 1;
  }
  *out = cache[dev];
  return hipSuccess;
}

template <int D, int PM, bool PAGED>
static hipError_t launch_prep_bf16(const KvPrepArgs& a, hipStream_t st) {
  constexpr int half = D / 2, RK = 64 / (half / (2 * kPrepKeyWords)), ND = D / 64;
  const int64_t nK = (int64_t)a.B * (a.Lp / RK) * ((a.Hkv + kPrepKeyHeads - 1) / kPrepKeyHeads);
  const int64_t nV = a.vt ? (int64_t)a.B * (a.Lp / kPrefillTileKeys) * a.Hkv * ND : 0;
  int resident = 0;
  const hipError_t e = resident_workgroups(kv_prep_bf16_kernel<D, PM, PAGED>, &resident);
  if (e != hipSuccess) return e;
  const int64_t need = (nK + nV + 3) / 4;
  int64_t grid = 2 * (int64_t)resident;
  if (grid > need) grid = need;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((kv_prep_bf16_kernel<D, PM, PAGED>), dim3((unsigned)grid), dim3(256), 0, st, a, nK, nV);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prep_bf16_d(const KvPrepArgs& a, hipStream_t st) {
  const bool paged = a.pg.bt != nullptr;
  if (a.pos_mode == 1) return paged ? launch_prep_bf16<D, 1, true>(a, st) : launch_prep_bf16<D, 1, false>(a, st);
  if (a.pos_mode == 2) return paged ? launch_prep_bf16<D, 2, true>(a, st) : launch_prep_bf16<D, 2, false>(a, st);
  return paged ? launch_prep_bf16<D, 0, true>(a, st) : launch_prep_bf16<D, 0, false>(a, st);
}

hipError_t launch_kv_prep(const KvPrepArgs& a, int dtype, hipStream_t st) {
  if (dtype == 0) {
    const dim3 grid((unsigned)(a.Lp / kPrefillTileKeys), (unsigned)a.Hkv, (unsigned)a.B);
    if (a.D == 64)
      hipLaunchKernelGGL((kv_prep_f32_kernel<64>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((kv_prep_f32_kernel<128>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  // the bf16 pass takes its angles from a.base or a.theta, never a table
  if (a.table != nullptr) return hipErrorInvalidValue;
  return a.D == 64 ? launch_prep_bf16_d<64>(a, st) : launch_prep_bf16_d<128>(a, st);
}

}  // namespace dca
