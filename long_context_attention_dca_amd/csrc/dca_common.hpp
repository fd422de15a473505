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

}  // namespace dca
