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

// ---- cos/sin table [npos][D/2] (fp64) ----------------------------------------------
__global__ void rope_table_kernel(double2* __restrict__ table, int npos, int half, int D, double base) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= npos * half) return;
  const int p = idx / half, k = idx - p * half;
  const double theta = pow(base, -2.0 * (double)k / (double)D);
  double sn, cs;
  sincos((double)p * theta, &sn, &cs);
  table[idx] = make_double2(cs, sn);
}

hipError_t launch_rope_table(double2* table, int npos, int D, double base, hipStream_t st) {
  const int half = D / 2;
  const int n = npos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, table, npos, half, D,
                     base);
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

__global__ void cf_query_table_kernel(double2* __restrict__ tab, int L, int half, int C, double inv_kappa,
                                      const double* __restrict__ theta) {
  const int i = blockIdx.x, cls = blockIdx.y, k = threadIdx.x;
  if (k < half) tab[((int64_t)cls * L + i) * half + k] = rope_cs(cf_query_pos(cls, i, C, inv_kappa), theta[k]);
}

hipError_t launch_cf_query_table(double2* tab, int L, int D, int C, double inv_kappa, const double* theta,
                                 hipStream_t st) {
  hipLaunchKernelGGL(cf_query_table_kernel, dim3(L, 3), dim3(64), 0, st, tab, L, D / 2, C, inv_kappa, theta);
  return hipGetLastError();
}

// ---- dca_rope_remap -----------------------------------------------------------------
// One workgroup per token t: the 64 (or 32) angles of its position are made
// once in fp64 and applied to every (batch, head) row of that token.
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

template <typename T>
__global__ void __launch_bounds__(256) rope_remap_kernel(const T* __restrict__ x, T* __restrict__ out,
                                                         int64_t B, int64_t L, int H, int D,
                                                         int64_t pos0, int map, int c, int w,
                                                         double base, double step) {
  __shared__ double2 cs[64];
  const int64_t t = blockIdx.x;
  const int half = D / 2;
  const int64_t p = pos0 + t;
  const double P = map == kRemapCoarseScaled ? (double)(p / c) * step + (double)(p % c)
                                             : (double)remap_position(p, map, c, w);
  if ((int)threadIdx.x < half) {
    const double theta = pow(base, -2.0 * (double)threadIdx.x / (double)D);
    double sn, cn;
    sincos(P * theta, &sn, &cn);
    cs[threadIdx.x] = make_double2(cn, sn);
  }
  __syncthreads();
  const int64_t per_b = (int64_t)H * half;
  for (int64_t idx = threadIdx.x; idx < B * per_b; idx += blockDim.x) {
    const int64_t b = idx / per_b;
    const int rem = (int)(idx - b * per_b);
    const int h = rem / half, k = rem - h * half;
    const int64_t off = ((b * L + t) * H + h) * D;
    const double x1 = Elem<T>::load(x + off + k);
    const double x2 = Elem<T>::load(x + off + k + half);
    const double2 a = cs[k];
    Elem<T>::store(out + off + k, (float)(x1 * a.x - x2 * a.y));
    Elem<T>::store(out + off + k + half, (float)(x2 * a.x + x1 * a.y));
  }
}

hipError_t launch_rope_remap(const void* x, void* out, int64_t B, int64_t L, int64_t H, int64_t D,
                             int64_t pos0, int map, int c, int w, double base, int dtype,
                             hipStream_t st, double step) {
  if (L == 0 || B == 0 || H == 0) return hipSuccess;
  if (dtype == 0)
    hipLaunchKernelGGL(rope_remap_kernel<float>, dim3((unsigned)L), dim3(256), 0, st,
                       (const float*)x, (float*)out, B, L, (int)H, (int)D, pos0, map, c, w, base, step);
  else
    hipLaunchKernelGGL(rope_remap_kernel<uint16_t>, dim3((unsigned)L), dim3(256), 0, st,
                       (const uint16_t*)x, (uint16_t*)out, B, L, (int)H, (int)D, pos0, map, c, w,
                       base, step);
  return hipGetLastError();
}

// ---- prefill K/V prep ---------------------------------------------------------------
// Within each 16-key group of a V^T tile the keys are stored in the order
// 0-3, 8-11, 4-7, 12-15 (bits 2 and 3 of the key index swapped).  That is the
// order in which one half-wave holds the probabilities of a 16-key step in the
// 32x32 MFMA output layout, so the PV step reads 8 contiguous keys per lane.
__device__ inline int vt_perm(int p) { return (p & ~15) | (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1); }

template <typename T, int D, bool TRANSPOSE_V>
__global__ void __launch_bounds__(256) kv_prep_kernel(KvPrepArgs a) {
  constexpr int half = D / 2;
  constexpr int TK = kPrefillTileKeys;
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int j0 = tile * TK;
  const int Lb = a.per_seq ? a.seq_len[b] : a.L;   // valid rows of this sequence
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const T* k = (const T*)a.k;
  T* krot = (T*)a.krot;
  T* k_rot_out = (T*)a.k_rot_out;
  for (int idx = threadIdx.x; idx < TK * half; idx += 256) {
    const int row = idx / half, kk = idx - row * half;
    const int j = j0 + row;
    T* dst = krot + (bg * a.Lp + j) * D;
    const int64_t crow = j < Lb ? cache_row(a.pg, a.in_rows, b, j) : 0;
    if (j < Lb && crow < 0) {   // unreadable page: poison the key so the rows using it give NaN
      Elem<T>::store(dst + kk, __builtin_nanf(""));
      Elem<T>::store(dst + kk + half, __builtin_nanf(""));
    } else if (j < Lb) {
      const int64_t in = (crow * a.Hkv + g) * D;
      const double x1 = Elem<T>::load(k + in + kk);
      const double x2 = Elem<T>::load(k + in + kk + half);
      if (a.table || a.pos_mode == 1) {
        const double2 c = a.pos_mode == 1
                              ? rope_cs((double)(j / a.cf_chunk) * a.cf_step + (double)(j % a.cf_chunk),
                                        a.theta[kk])
                              : a.table[((j / a.kdiv) % a.kmod) * half + kk];
        const float y1 = (float)(x1 * c.x - x2 * c.y);
        const float y2 = (float)(x2 * c.x + x1 * c.y);
        Elem<T>::store(dst + kk, y1);
        Elem<T>::store(dst + kk + half, y2);
        if (k_rot_out) {
          Elem<T>::store(k_rot_out + in + kk, y1);
          Elem<T>::store(k_rot_out + in + kk + half, y2);
        }
      } else {   // already rotated: exact copy
        Elem<T>::store(dst + kk, (float)x1);
        Elem<T>::store(dst + kk + half, (float)x2);
      }
    } else {
      Elem<T>::store(dst + kk, 0.f);
      Elem<T>::store(dst + kk + half, 0.f);
    }
  }
  if constexpr (TRANSPOSE_V) {
    if (a.vt == nullptr) return;   // uniform: a second key rotation without V
    __shared__ uint16_t vs[TK][D + 2];
    const uint16_t* vv = reinterpret_cast<const uint16_t*>(a.v);
    for (int idx = threadIdx.x; idx < TK * D; idx += 256) {
      const int row = idx / D, d = idx - row * D;
      const int j = j0 + row;
      const int64_t crow = j < Lb ? cache_row(a.pg, a.in_rows, b, j) : -1;
      vs[row][d] = crow >= 0 ? vv[(crow * a.Hkv + g) * D + d] : (uint16_t)0;
    }
    __syncthreads();
    const int ntiles = a.Lp / TK;
    uint16_t* dst = (uint16_t*)a.vt + ((bg * ntiles + tile) * D) * TK;
    for (int idx = threadIdx.x; idx < D * TK; idx += 256) {
      const int d = idx / TK, p = idx - d * TK;
      dst[idx] = vs[vt_perm(p)][d];
    }
  }
}

hipError_t launch_kv_prep(const KvPrepArgs& a, int dtype, hipStream_t st) {
  const dim3 grid((unsigned)(a.Lp / kPrefillTileKeys), (unsigned)a.Hkv, (unsigned)a.B);
  if (dtype == 0) {
    if (a.D == 64)
      hipLaunchKernelGGL((kv_prep_kernel<float, 64, false>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((kv_prep_kernel<float, 128, false>), grid, dim3(256), 0, st, a);
  } else {
    if (a.D == 64)
      hipLaunchKernelGGL((kv_prep_kernel<uint16_t, 64, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((kv_prep_kernel<uint16_t, 128, true>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dca
