// dca_common.hpp - device helpers shared by the DCA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- position maps ---------------------------------------------------------
// Chunk size s = c - w.  Keys sit at j mod s; a query's position depends on
// the chunk relation rho = floor(i/s) - floor(j/s) of the pair:
//   rho = 0 -> i mod s, rho = 1 -> min(s + i mod s, c - 1), rho >= 2 -> c - 1.
// `cls` below is min(rho, 2).
__host__ __device__ inline int query_pos(int cls, int r, int s, int c) {
  if (cls == 0) return r;
  if (cls == 1) return (s + r < c) ? s + r : c - 1;
  return c - 1;
}

// SelfExtend ("LLM Maybe LongLM", abstract: grouped attention for distant
// tokens, neighbor attention inside a window W).  Neighbor pairs (i - j < W)
// keep positions i and j; grouped pairs put key j at floor(j / G) and query i
// at floor(i / G) + W - floor(W / G), so their distance is at least W.
__host__ __device__ inline int se_query_pos_grouped(int i, int G, int W) { return i / G + W - W / G; }

// The DCA guide's coarse / fine distances ("Inter-Chunk Attention" and
// "Successive Chunk Smoothing") factor into query minus key positions, with
// chunk size C, offset o = x mod C and kappa = L_target / L_train:
//   keys:    plain j (same or adjacent chunk), floor(j/C) C / kappa + o_j (older)
//   queries: i (same chunk), i - o_i (1 - 1/kappa) (adjacent), floor(i/C) C / kappa + o_i.
// Positions are real numbers (fp64).
__host__ __device__ inline double cf_query_pos(int cls, int i, int C, double inv_kappa) {
  const int o = i % C;
  if (cls == 0) return (double)i;
  if (cls == 1) return (double)i - (double)o * (1.0 - inv_kappa);
  return (double)(i / C) * (double)C * inv_kappa + (double)o;
}

// sin and cos in fp64 without a library call (inlined, no stack): Cody-Waite
// reduction x = n (pi/2) + r with pi/2 split into three parts (the first two
// hold 33 significant bits each, so n * part is exact for n < 2^20; fma keeps
// the reduction accurate beyond), then Taylor series on |r| <= pi/4 up to
// r^17 / r^18 (truncation below 1e-19).  The split was computed from pi to
// 130 digits (Machin's formula).  Used for RoPE angles of real-valued
// positions.
__host__ __device__ inline void dca_sincos(double x, double* s, double* c) {
  constexpr double kTwoOverPi = 0.6366197723675814;
  constexpr double kP1 = 1.5707963267341256;       // pi/2, first 33 bits
  constexpr double kP2 = 6.077100506303966e-11;    // next 33 bits
  constexpr double kP3 = 2.0222662487959506e-21;   // remainder
  const double n = rint(x * kTwoOverPi);
  double r = fma(-n, kP1, x);
  r = fma(-n, kP2, r);
  r = fma(-n, kP3, r);
  const double r2 = r * r;
  // 1/k! for the odd (sin) and even (cos) terms, Horner from the highest
  constexpr double f3 = 1.0 / 6.0, f5 = f3 / 20.0, f7 = f5 / 42.0, f9 = f7 / 72.0, f11 = f9 / 110.0,
                   f13 = f11 / 156.0, f15 = f13 / 210.0, f17 = f15 / 272.0;
  constexpr double f2 = 0.5, f4 = f2 / 12.0, f6 = f4 / 30.0, f8 = f6 / 56.0, f10 = f8 / 90.0,
                   f12 = f10 / 132.0, f14 = f12 / 182.0, f16 = f14 / 240.0, f18 = f16 / 306.0;
  double ps = -f17;
  ps = fma(ps, r2, f15);
  ps = fma(ps, r2, -f13);
  ps = fma(ps, r2, f11);
  ps = fma(ps, r2, -f9);
  ps = fma(ps, r2, f7);
  ps = fma(ps, r2, -f5);
  ps = fma(ps, r2, f3);
  const double sr = fma(-ps * r2, r, r);          // r - r^3/3! + ...
  double pc = f18;
  pc = fma(pc, r2, -f16);
  pc = fma(pc, r2, f14);
  pc = fma(pc, r2, -f12);
  pc = fma(pc, r2, f10);
  pc = fma(pc, r2, -f8);
  pc = fma(pc, r2, f6);
  pc = fma(pc, r2, -f4);
  pc = fma(pc, r2, f2);
  const double cr = fma(-pc, r2, 1.0);            // 1 - r^2/2! + ...
  const long long q = (long long)n & 3;
  if (q == 0) {
    *s = sr;
    *c = cr;
  } else if (q == 1) {
    *s = cr;
    *c = -sr;
  } else if (q == 2) {
    *s = -sr;
    *c = -cr;
  } else {
    *s = -cr;
    *c = sr;
  }
}

// cos / sin of a real position p times theta_k (theta from a precomputed
// table, so no library call is made), in fp64.
__device__ inline double2 rope_cs(double p, double theta) {
  double sn, cs;
  dca_sincos(p * theta, &sn, &cs);
  return make_double2(cs, sn);
}

// ---- bf16 <-> fp32 -----------------------------------------------------------
__device__ inline float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest even (the hardware conversion on gfx950).
__device__ inline uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Lane l and lane l ^ 32 combined, in every lane (v_permlane32_swap: no LDS
// round trip).  Component 0 holds the low half's value in lanes 0-31 and
// 32-63 alike after the swap, component 1 the high half's.
__device__ inline float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline void unpack_bf16x8(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ inline uint4 pack_bf16x8(const float* f) {
  uint4 u;
  u.x = pack_bf16x2(f[0], f[1]);
  u.y = pack_bf16x2(f[2], f[3]);
  u.z = pack_bf16x2(f[4], f[5]);
  u.w = pack_bf16x2(f[6], f[7]);
  return u;
}

// 16-byte global load with the non-temporal hint (the `nt` bit): for data
// streamed through once, which is then not kept in L2 / MALL.  A plain read
// of a 6.55 GB buffer measured 6.1 TB/s, the same read with the hint
// 6.7-6.8 TB/s.
__device__ inline uint4 load_stream(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(t[0], t[1], t[2], t[3]);
}
// 16-byte global store with the non-temporal hint, for output that is not
// read again soon.
__device__ inline void store_stream(uint4* p, const uint4& v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 t;
  t[0] = v.x;
  t[1] = v.y;
  t[2] = v.z;
  t[3] = v.w;
  __builtin_nontemporal_store(t, (u32x4*)p);
}
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float x) { *p = x; }
};
template <>
struct Elem<uint16_t> {
  __device__ static float load(const uint16_t* p) { return bf2f(*p); }
  __device__ static void store(uint16_t* p, float x) { *p = f2bf(x); }
};

// Cache row of key j of sequence b: dense [B, rows, ...] or paged (the row
// inside the page pool).  -1 when the block-table entry lies outside the pool;
// callers then read nothing and poison what they produce with NaN.
template <typename PG>
__device__ inline int64_t cache_row(const PG& pg, int64_t dense_rows, int b, int j) {
  if (!pg.bt) return (int64_t)b * dense_rows + j;
  const int page = pg.bt[(int64_t)b * pg.max_blocks + j / pg.page_size];
  return (page >= 0 && page < pg.num_pages) ? (int64_t)page * pg.page_size + j % pg.page_size : -1;
}

}  // namespace dca
