// abi.hip - the extern "C" entry points declared in include/dca.h.
//
// Every argument is validated on the host before the first HIP call, so an
// invalid call returns its status without touching the device.  Scratch space
// is carved from the caller's workspace; the library allocates nothing and
// keeps no state between calls.
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "dca.h"
#include "dca_launch.hpp"

using namespace dca;

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;  // per-dimension bound (grid sizes, int indices)

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool dtype_ok(int dtype) { return dtype == DCA_F32 || dtype == DCA_BF16; }
bool head_dim_ok(int64_t D) { return D == 64 || D == 128; }
int64_t elem_size(int dtype) { return dtype == DCA_F32 ? 4 : 2; }
bool cw_ok(int c, int w) { return c >= 1 && c <= (1 << 24) && w >= 0 && w < c; }
// Sizes of the prefill family: B and Hkv index grid dimensions limited to
// 65535, and the padded K (or V) copy must stay far inside size_t.  One
// head's padded key (or value) rows, Lp * D elements, must stay below 2^31
// bytes: the attention kernel addresses a head through one buffer resource
// whose record count and per-tile offsets are 32-bit (bf16 at D = 128: at
// most 2^23 - 128 tokens; D = 64: 2^24 - 128).
constexpr int64_t kMaxGridYZ = 65535;
constexpr int64_t kMaxHeadBytes = int64_t(1) << 31;
bool prefill_sizes_ok(int64_t B, int64_t L, int64_t Hkv, int64_t D, int dtype) {
  if (B > kMaxGridYZ || Hkv > kMaxGridYZ || L >= kMaxDim / 2) return false;
  if (round_up(L, kPrefillRowAlign) * D * elem_size(dtype) >= kMaxHeadBytes) return false;
  return (double)B * (double)Hkv * (double)round_up(L, kPrefillRowAlign) * (double)D * 4.0 < 0x1p56;
}
bool base_ok(double base) { return base > 0.0 && isfinite(base); }

struct PrefillLayout {
  int64_t Lp;
  size_t table, krot, vt, total;
};

bool prefill_layout(int64_t B, int64_t L, int64_t Hkv, int64_t D, int c, int dtype,
                    PrefillLayout* out) {
  if (B < 1 || L < 1 || Hkv < 1 || !head_dim_ok(D) || !dtype_ok(dtype) || c < 1) return false;
  if (!prefill_sizes_ok(B, L, Hkv, D, dtype)) return false;
  PrefillLayout p;
  p.Lp = round_up(L, kPrefillRowAlign);
  const int64_t tbytes = (int64_t)c * (D / 2) * 16;
  const int64_t kbytes = B * Hkv * p.Lp * D * elem_size(dtype);
  const int64_t vbytes = B * Hkv * p.Lp * D * elem_size(dtype);
  p.table = 0;
  p.krot = (size_t)round_up(tbytes, 256);
  p.vt = p.krot + (size_t)round_up(kbytes, 256);
  p.total = p.vt + (size_t)round_up(vbytes, 256);
  *out = p;
  return true;
}

// SelfExtend workspace: fp64 cos/sin table for positions [0, npos) | keys at j
// | keys at floor(j / G) | V (bf16: tiled transpose; fp32: copy).
bool se_ok(int64_t G, int64_t W) { return G >= 1 && G <= (1 << 24) && W >= 0 && W <= (1 << 30); }

struct SeLayout {
  int64_t Lp, npos;
  size_t table, krot, krot2, vt, total;
};

bool se_layout(int64_t B, int64_t L, int64_t Hkv, int64_t D, int G, int W, int dtype, SeLayout* out) {
  if (B < 1 || L < 1 || Hkv < 1 || !head_dim_ok(D) || !dtype_ok(dtype) || !se_ok(G, W)) return false;
  if (!prefill_sizes_ok(B, L, Hkv, D, dtype)) return false;
  SeLayout p;
  p.Lp = round_up(L, kPrefillRowAlign);
  // largest position used: L - 1 (neighbor query) or the grouped query of row L - 1
  const int64_t top_grouped = (L - 1) / G + W - W / G;
  p.npos = (top_grouped > L - 1 ? top_grouped : L - 1) + 1;
  if (p.npos >= kMaxDim / 64) return false;
  const int64_t tbytes = p.npos * (D / 2) * 16;
  const int64_t kbytes = B * Hkv * p.Lp * D * elem_size(dtype);
  p.table = 0;
  p.krot = (size_t)round_up(tbytes, 256);
  p.krot2 = p.krot + (size_t)round_up(kbytes, 256);
  p.vt = p.krot2 + (size_t)round_up(kbytes, 256);
  p.total = p.vt + (size_t)round_up(kbytes, 256);
  *out = p;
  return true;
}

struct DecodeLayout {
  int kps, ns;
  size_t qv, part_o, part_lse, total;
};

// kv: per-sequence cached key counts (host), or null for B sequences of
// kv_len keys; kv_len is the longest sequence either way.
bool decode_layout(int64_t B, const int64_t* kv, int64_t kv_len, int64_t Hq, int64_t Hkv, int64_t D, int dtype,
                   DecodeLayout* out) {
  if (B < 1 || kv_len < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || !head_dim_ok(D) || !dtype_ok(dtype))
    return false;
  if (B >= kMaxDim || kv_len >= kMaxDim / 2 || Hq >= 65536 || B * Hq >= kMaxDim) return false;
  DecodeLayout p;
  decode_plan(kv, B, kv_len, Hq, Hkv, dtype, &p.kps, &p.ns);
  p.qv = 0;
  p.part_o = (size_t)round_up(B * Hq * 3 * D * elem_size(dtype), 256);
  p.part_lse = p.part_o + (size_t)round_up(B * Hq * (int64_t)p.ns * D * 4, 256);
  p.total = p.part_lse + (size_t)round_up(B * Hq * (int64_t)p.ns * 4, 256);
  *out = p;
  return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DCA_OK : DCA_ERR_HIP; }

}  // namespace

extern "C" {

const char* dca_status_string(int status) {
  switch (status) {
    case DCA_OK:
      return "DCA_OK: success (work enqueued)";
    case DCA_ERR_INVALID_ARG:
      return "DCA_ERR_INVALID_ARG: null pointer, bad shape, w >= c, Hq % Hkv != 0 or misaligned pointer";
    case DCA_ERR_UNSUPPORTED:
      return "DCA_ERR_UNSUPPORTED: head dim must be 64 or 128 and dtype DCA_F32 or DCA_BF16";
    case DCA_ERR_WORKSPACE:
      return "DCA_ERR_WORKSPACE: workspace missing, misaligned or smaller than the size query";
    case DCA_ERR_HIP:
      return "DCA_ERR_HIP: a HIP launch reported an error";
    case DCA_ERR_TOO_LARGE:
      return "DCA_ERR_TOO_LARGE: the call needs more scratch than the library's static buffer holds";
    default:
      return "unknown DCA status";
  }
}

int dca_version(void) { return 10000; }

int dca_rope_remap(const void* x, void* out, int64_t B, int64_t L, int64_t H, int64_t D, int64_t pos0,
                   int map, int c, int w, double rope_base, int dtype, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!x || !out || B < 0 || L < 0 || H < 0 || pos0 < 0) return DCA_ERR_INVALID_ARG;
  if (B >= kMaxDim || L >= kMaxDim || H * D >= kMaxDim || pos0 > (int64_t(1) << 52)) return DCA_ERR_INVALID_ARG;
  const bool se_map = map == DCA_MAP_SE_KEY_GROUPED || map == DCA_MAP_SE_Q_GROUPED;
  if (map < DCA_MAP_KEY || map > DCA_MAP_SE_Q_GROUPED || !base_ok(rope_base)) return DCA_ERR_INVALID_ARG;
  if (se_map ? !se_ok(c, w) : !cw_ok(c, w)) return DCA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(out, 16)) return DCA_ERR_INVALID_ARG;
  if (B == 0 || L == 0 || H == 0) return DCA_OK;
  return hip_status(launch_rope_remap(x, out, B, L, H, D, pos0, map, c, w, rope_base, dtype,
                                      (hipStream_t)stream));
}

size_t dca_prefill_workspace_bytes(int64_t B, int64_t L, int64_t Hkv, int64_t D, int c, int dtype) {
  PrefillLayout p;
  return prefill_layout(B, L, Hkv, D, c, dtype, &p) ? p.total : 0;
}

static int prefill_common_checks(int64_t B, int64_t L, int64_t Hkv, int64_t D, int c, int w,
                                 int dtype, const void* ws, size_t ws_bytes, PrefillLayout* p) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (B < 1 || L < 1 || Hkv < 1 || !cw_ok(c, w)) return DCA_ERR_INVALID_ARG;
  if (!prefill_layout(B, L, Hkv, D, c, dtype, p)) return DCA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p->total || !aligned(ws, 256)) return DCA_ERR_WORKSPACE;
  return DCA_OK;
}

static int prepare_impl(const void* k, const void* v, void* k_rot_out, int64_t B, int64_t L,
                        int64_t Hkv, int64_t D, int c, int w, double rope_base, int dtype,
                        void* ws, const PrefillLayout& p, hipStream_t st) {
  uint8_t* base = (uint8_t*)ws;
  double2* table = (double2*)(base + p.table);
  hipError_t e = hipSuccess;
  KvPrepArgs kp = {};
  kp.k = k;
  kp.v = v;
  if (dtype == DCA_BF16) {
    // one launch: keys turned with cos / sin made in the kernel, and the
    // query cos / sin table (fp32) written beside them
    kp.table = nullptr;
    kp.pos_mode = 2;
    kp.base = rope_base;
    kp.table_out = (float2*)table;
    kp.table_rows = c;
  } else {
    e = launch_rope_table(table, c, (int)D, rope_base, false, st);   // the key pass reads rows
    if (e != hipSuccess) return DCA_ERR_HIP;
    kp.table = table;
  }
  kp.krot = base + p.krot;
  kp.vt = base + p.vt;
  kp.k_rot_out = k_rot_out;
  kp.B = (int)B;
  kp.in_rows = (int)L;
  kp.L = (int)L;
  kp.Lp = (int)p.Lp;
  kp.Hkv = (int)Hkv;
  kp.D = (int)D;
  kp.kdiv = 1;
  kp.kmod = c - w;
  e = launch_kv_prep(kp, dtype, st);
  if (e != hipSuccess) return DCA_ERR_HIP;
  if (dtype == DCA_F32) {
    e = hipMemcpyAsync(base + p.vt, v, (size_t)(B * L * Hkv * D * 4), hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return DCA_ERR_HIP;
  }
  return DCA_OK;
}

static int attend_impl(const void* q, void* o, float* lse, int64_t B, int64_t L, int64_t Hq,
                       int64_t Hkv, int64_t D, int c, int w, float sm_scale, int dtype,
                       const void* ws, const PrefillLayout& p, hipStream_t st) {
  const uint8_t* base = (const uint8_t*)ws;
  PrefillArgs a = {};
  a.q = q;
  a.krot = base + p.krot;
  a.vt = base + p.vt;
  // bf16: the prepare launch wrote it in fp32, frequency-major; fp32: fp64, row-major
  if (dtype == DCA_BF16) {
    a.ftable = (const float2*)(base + p.table);
    a.tab_ps = 1;
    a.tab_ks = c;
  } else {
    a.table = (const double2*)(base + p.table);
    a.tab_ps = D / 2;
    a.tab_ks = 1;
  }
  a.o = o;
  a.lse = lse;
  a.B = (int)B;
  a.L = (int)L;
  a.Lp = (int)p.Lp;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.D = (int)D;
  a.c = c;
  a.w = w;
  a.s = c - w;
  a.map = kMapDCA;
  a.krot2 = nullptr;
  a.se_group = 1;
  a.se_window = 0;
  a.q_rows = (int)L;
  a.per_seq = 0;
  a.v_rows = (int)L;
  a.sm_scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)D));
  return hip_status(dtype == DCA_BF16 ? launch_prefill_bf16(a, st) : launch_prefill_f32(a, st));
}

static bool attend_args_ok(const void* q, const void* o, const float* lse, int64_t B, int64_t L,
                           int64_t Hq, int64_t Hkv, float sm_scale) {
  if (!q || !o || Hq < 1 || Hkv < 1 || Hq % Hkv || Hq >= 65536) return false;
  if (B * Hq * ((L + 127) / 128) >= kMaxDim || !isfinite(sm_scale)) return false;
  return aligned(q, 16) && aligned(o, 16) && (!lse || aligned(lse, 4));
}

int dca_prefill_prepare(const void* k, const void* v, void* k_rot_out, int64_t B, int64_t L,
                        int64_t Hkv, int64_t D, int c, int w, double rope_base, int dtype,
                        void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16) || (k_rot_out && !aligned(k_rot_out, 16)) ||
      !base_ok(rope_base))
    return DCA_ERR_INVALID_ARG;
  PrefillLayout p;
  const int r = prefill_common_checks(B, L, Hkv, D, c, w, dtype, ws, ws_bytes, &p);
  if (r != DCA_OK) return r;
  return prepare_impl(k, v, k_rot_out, B, L, Hkv, D, c, w, rope_base, dtype, ws, p,
                      (hipStream_t)stream);
}

int dca_prefill_attend(const void* q, void* o, float* lse, int64_t B, int64_t L, int64_t Hq,
                       int64_t Hkv, int64_t D, int c, int w, float sm_scale, int dtype,
                       const void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!attend_args_ok(q, o, lse, B, L, Hq, Hkv, sm_scale)) return DCA_ERR_INVALID_ARG;
  PrefillLayout p;
  const int r = prefill_common_checks(B, L, Hkv, D, c, w, dtype, ws, ws_bytes, &p);
  if (r != DCA_OK) return r;
  return attend_impl(q, o, lse, B, L, Hq, Hkv, D, c, w, sm_scale, dtype, ws, p,
                     (hipStream_t)stream);
}

int dca_prefill(const void* q, const void* k, const void* v, void* o, float* lse, void* k_rot_out,
                int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int c, int w,
                double rope_base, float sm_scale, int dtype, void* ws, size_t ws_bytes,
                void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16) || (k_rot_out && !aligned(k_rot_out, 16)) ||
      !base_ok(rope_base) || !attend_args_ok(q, o, lse, B, L, Hq, Hkv, sm_scale))
    return DCA_ERR_INVALID_ARG;
  PrefillLayout p;
  const int r = prefill_common_checks(B, L, Hkv, D, c, w, dtype, ws, ws_bytes, &p);
  if (r != DCA_OK) return r;
  hipStream_t st = (hipStream_t)stream;
  const int rp = prepare_impl(k, v, k_rot_out, B, L, Hkv, D, c, w, rope_base, dtype, ws, p, st);
  if (rp != DCA_OK) return rp;
  return attend_impl(q, o, lse, B, L, Hq, Hkv, D, c, w, sm_scale, dtype, ws, p, st);
}

size_t dca_selfextend_workspace_bytes(int64_t B, int64_t L, int64_t Hkv, int64_t D, int group,
                                      int window, int dtype) {
  SeLayout p;
  return se_layout(B, L, Hkv, D, group, window, dtype, &p) ? p.total : 0;
}

int dca_selfextend_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int group,
                           int window, double rope_base, float sm_scale, int dtype, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16) || !base_ok(rope_base) ||
      !attend_args_ok(q, o, lse, B, L, Hq, Hkv, sm_scale))
    return DCA_ERR_INVALID_ARG;
  if (B < 1 || L < 1 || !se_ok(group, window)) return DCA_ERR_INVALID_ARG;
  SeLayout p;
  if (!se_layout(B, L, Hkv, D, group, window, dtype, &p)) return DCA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.total || !aligned(ws, 256)) return DCA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)ws;
  double2* table = (double2*)(base + p.table);
  // neighbor keys at j (with the V layout), grouped keys at floor(j / G)
  const int unbounded = 1 << 30;
  KvPrepArgs kp = {};
  kp.k = k;
  kp.v = v;
  if (dtype == DCA_BF16) {
    // keys turned with cos / sin made in the kernel; the first launch also
    // writes the query cos / sin table (fp32, frequency-major)
    kp.pos_mode = 2;
    kp.base = rope_base;
    kp.table_out = (float2*)table;
    kp.table_rows = (int)p.npos;
  } else {
    if (launch_rope_table(table, (int)p.npos, (int)D, rope_base, false, st) != hipSuccess) return DCA_ERR_HIP;
    kp.table = table;
  }
  kp.krot = base + p.krot;
  kp.vt = base + p.vt;
  kp.B = (int)B;
  kp.in_rows = (int)L;
  kp.L = (int)L;
  kp.Lp = (int)p.Lp;
  kp.Hkv = (int)Hkv;
  kp.D = (int)D;
  kp.kdiv = 1;
  kp.kmod = unbounded;
  if (launch_kv_prep(kp, dtype, st) != hipSuccess) return DCA_ERR_HIP;
  kp.krot = base + p.krot2;
  kp.vt = nullptr;
  kp.kdiv = group;
  kp.table_out = nullptr;
  if (launch_kv_prep(kp, dtype, st) != hipSuccess) return DCA_ERR_HIP;
  if (dtype == DCA_F32 &&
      hipMemcpyAsync(base + p.vt, v, (size_t)(B * L * Hkv * D * 4), hipMemcpyDeviceToDevice, st) != hipSuccess)
    return DCA_ERR_HIP;
  PrefillArgs a = {};
  a.q = q;
  a.krot = base + p.krot;
  a.krot2 = base + p.krot2;
  a.vt = base + p.vt;
  if (dtype == DCA_BF16) {
    a.ftable = (const float2*)table;
    a.tab_ps = 1;   // frequency-major
    a.tab_ks = p.npos;
  } else {
    a.table = table;
    a.tab_ps = D / 2;   // row-major: the key passes read it too
    a.tab_ks = 1;
  }
  a.o = o;
  a.lse = lse;
  a.B = (int)B;
  a.L = (int)L;
  a.Lp = (int)p.Lp;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.D = (int)D;
  // DCA fields unused: one chunk as long as any sequence
  a.c = unbounded;
  a.w = 0;
  a.s = unbounded;
  a.map = kMapSelfExtend;
  a.se_group = group;
  a.se_window = window;
  a.q_rows = (int)L;
  a.per_seq = 0;
  a.v_rows = (int)L;
  a.sm_scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)D));
  return hip_status(dtype == DCA_BF16 ? launch_prefill_bf16(a, st) : launch_prefill_f32(a, st));
}

// Coarse / fine map workspace: theta_k table (512 B) | (cos, sin) of the three
// query positions of every row, [3][L][D/2] double2 | keys at their plain
// positions | keys at the coarse-scaled positions | V (bf16: tiled transpose;
// fp32: unused).
constexpr size_t kThetaBytes = 512;   // D/2 <= 64 doubles

struct CfLayout {
  int64_t Lp;
  size_t qtab, krot, krot2, vt, total;
};

static bool cf_layout(int64_t B, int64_t L, int64_t Hkv, int64_t D, int dtype, CfLayout* p) {
  if (B < 1 || L < 1 || Hkv < 1 || !head_dim_ok(D) || !dtype_ok(dtype)) return false;
  if (!prefill_sizes_ok(B, L, Hkv, D, dtype)) return false;
  p->Lp = round_up(L, kPrefillRowAlign);
  const int64_t kbytes = round_up(B * Hkv * p->Lp * D * elem_size(dtype), 256);
  p->qtab = kThetaBytes;
  p->krot = p->qtab + (size_t)round_up(3 * L * (D / 2) * 16, 256);
  p->krot2 = p->krot + (size_t)kbytes;
  p->vt = p->krot2 + (size_t)kbytes;
  p->total = p->vt + (size_t)kbytes;
  return true;
}

size_t dca_coarse_fine_workspace_bytes(int64_t B, int64_t L, int64_t Hkv, int64_t D, int dtype) {
  CfLayout p;
  return cf_layout(B, L, Hkv, D, dtype, &p) ? p.total : 0;
}

int dca_coarse_fine_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                            int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int chunk, int train_len,
                            int target_len, double rope_base, float sm_scale, int dtype, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16) || !base_ok(rope_base) ||
      !attend_args_ok(q, o, lse, B, L, Hq, Hkv, sm_scale))
    return DCA_ERR_INVALID_ARG;
  if (chunk < 1 || chunk > (1 << 24) || train_len < 1 || target_len < 1) return DCA_ERR_INVALID_ARG;
  // bf16 runs the two-group kernel: every 32-row block and 64-key tile inside one chunk
  if (dtype == DCA_BF16 && chunk % kPrefillTileKeys != 0) return DCA_ERR_UNSUPPORTED;
  CfLayout p;
  if (!cf_layout(B, L, Hkv, D, dtype, &p)) return DCA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.total || !aligned(ws, 256)) return DCA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)ws;
  const double inv_kappa = (double)train_len / (double)target_len;
  double* theta = (double*)base;
  if (launch_rope_theta(theta, (int)D, rope_base, st) != hipSuccess) return DCA_ERR_HIP;
  // query cos / sin, frequency-major: fp32 for the bf16 kernel, fp64 for the fp32 one
  double2* qtab = (double2*)(base + p.qtab);
  if ((dtype == DCA_BF16 ? launch_cf_query_table_f32((float2*)qtab, (int)L, (int)D, chunk, inv_kappa, theta, st)
                         : launch_cf_query_table(qtab, (int)L, (int)D, chunk, inv_kappa, theta, st)) != hipSuccess)
    return DCA_ERR_HIP;
  // keys at plain positions (with the V layout), then at coarse-scaled positions
  KvPrepArgs kp = {};
  kp.k = k;
  kp.v = v;
  kp.table = nullptr;
  kp.krot = base + p.krot;
  kp.vt = dtype == DCA_BF16 ? base + p.vt : nullptr;
  kp.B = (int)B;
  kp.in_rows = (int)L;
  kp.L = (int)L;
  kp.Lp = (int)p.Lp;
  kp.Hkv = (int)Hkv;
  kp.D = (int)D;
  kp.kdiv = 1;
  kp.kmod = 1 << 30;
  kp.pos_mode = 1;
  kp.cf_chunk = chunk;
  kp.cf_step = (double)chunk;
  kp.theta = theta;
  if (launch_kv_prep(kp, dtype, st) != hipSuccess) return DCA_ERR_HIP;
  kp.krot = base + p.krot2;
  kp.vt = nullptr;
  kp.cf_step = (double)chunk * inv_kappa;
  if (launch_kv_prep(kp, dtype, st) != hipSuccess) return DCA_ERR_HIP;
  PrefillArgs a = {};
  a.q = q;
  a.krot = base + p.krot;
  a.krot2 = base + p.krot2;
  a.vt = dtype == DCA_BF16 ? (const void*)(base + p.vt) : v;   // fp32 reads V as given
  if (dtype == DCA_BF16)
    a.ftable = (const float2*)qtab;
  else
    a.table = qtab;
  a.tab_ps = 1;   // frequency-major over the 3 L query positions
  a.tab_ks = 3 * L;
  a.o = o;
  a.lse = lse;
  a.B = (int)B;
  a.L = (int)L;
  a.Lp = (int)p.Lp;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.D = (int)D;
  a.c = chunk;   // the chunk relation uses chunk size C (held in c and s)
  a.w = 0;
  a.s = chunk;
  a.map = kMapCoarseFine;
  a.se_group = 1;
  a.q_rows = (int)L;
  a.per_seq = 0;
  a.v_rows = (int)L;
  a.sm_scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)D));
  return hip_status(dtype == DCA_BF16 ? launch_prefill_bf16(a, st) : launch_prefill_f32(a, st));
}

size_t dca_decode_workspace_bytes(int64_t B, int64_t kv_len, int64_t Hq, int64_t Hkv, int64_t D,
                                  int dtype) {
  DecodeLayout p;
  return decode_layout(B, nullptr, kv_len, Hq, Hkv, D, dtype, &p) ? p.total : 0;
}

int dca_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
               int64_t B, int64_t kv_len, int64_t Hq, int64_t Hkv, int64_t D, int c, int w,
               double rope_base, float sm_scale, int dtype, void* ws, size_t ws_bytes,
               void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !o) return DCA_ERR_INVALID_ARG;
  if (B < 1 || kv_len < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return DCA_ERR_INVALID_ARG;
  if (!cw_ok(c, w) || !base_ok(rope_base) || !isfinite(sm_scale)) return DCA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return DCA_ERR_INVALID_ARG;
  DecodeLayout p;
  if (!decode_layout(B, nullptr, kv_len, Hq, Hkv, D, dtype, &p)) return DCA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.total || !aligned(ws, 256)) return DCA_ERR_WORKSPACE;

  uint8_t* base = (uint8_t*)ws;
  DecodeArgs a = {};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.o = o;
  a.lse = lse;
  a.qv = base + p.qv;
  a.part_o = (float*)(base + p.part_o);
  a.part_lse = (float*)(base + p.part_lse);
  a.B = (int)B;
  a.kv_len = (int)kv_len;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.D = (int)D;
  a.c = c;
  a.w = w;
  a.s = c - w;
  a.base = rope_base;
  a.sm_scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)D));
  a.keys_per_split = p.kps;
  a.nsplit = p.ns;
  a.cache_len = (int)kv_len;
  a.per_seq = 0;
  return hip_status(launch_decode(a, dtype, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Chunked prefill over a dense cache (pg.bt null; cache_len rows per
// sequence) or a paged one (cache_len = the most rows a sequence's table
// covers).  Arguments are validated here.
int prefill_chunk_impl(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                       const int64_t* pos0, const int64_t* q_len, int64_t B, int64_t Lq, int64_t cache_len,
                       int64_t Hq, int64_t Hkv, int64_t D, int c, int w, double rope_base, float sm_scale,
                       int dtype, void* ws, size_t ws_bytes, void* stream, const PagedKv& pg) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!k_cache || !v_cache || !pos0 || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !base_ok(rope_base) || !cw_ok(c, w) || !attend_args_ok(q, o, lse, B, Lq, Hq, Hkv, sm_scale))
    return DCA_ERR_INVALID_ARG;
  if (B < 1 || Lq < 1 || cache_len < 1 || cache_len >= kMaxDim / 2 || (!pg.bt && Lq > cache_len))
    return DCA_ERR_INVALID_ARG;
  // per-sequence offsets and lengths (host memory, read here)
  int64_t max_keys = 0, rows = 0;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t n = q_len ? q_len[b] : Lq;
    if (pos0[b] < 0 || n < 0 || n > Lq || pos0[b] + n > cache_len) return DCA_ERR_INVALID_ARG;
    max_keys = pos0[b] + n > max_keys ? pos0[b] + n : max_keys;
    rows += n;
  }
  if (rows == 0) return DCA_OK;   // no sequence has a row: nothing to do
  PrefillLayout p;
  if (!prefill_layout(B, max_keys, Hkv, D, c, dtype, &p)) return DCA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.total || !aligned(ws, 256)) return DCA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)ws;
  // query cos / sin, frequency-major: fp32 for the bf16 kernel, fp64 for the fp32 one
  double2* table = (double2*)(base + p.table);
  if ((dtype == DCA_BF16 ? launch_rope_table_f32((float2*)table, c, (int)D, rope_base, st)
                         : launch_rope_table(table, c, (int)D, rope_base, true, st)) != hipSuccess)
    return DCA_ERR_HIP;
  const int64_t es = elem_size(dtype);
  const int64_t kv_seq = cache_len * Hkv * D * es;    // bytes of one sequence's cache
  const int64_t ws_seq = Hkv * p.Lp * D * es;         // bytes of one sequence's tiles
  for (int64_t b0 = 0; b0 < B; b0 += kMaxSeqGroup) {
    const int nb = (int)(B - b0 < kMaxSeqGroup ? B - b0 : kMaxSeqGroup);
    // copy the cached (already rotated) keys and the values into the tiles
    KvPrepArgs kp = {};
    kp.k = (const uint8_t*)k_cache + (pg.bt ? 0 : b0 * kv_seq);
    kp.v = (const uint8_t*)v_cache + (pg.bt ? 0 : b0 * kv_seq);
    kp.pg = pg;
    if (pg.bt) kp.pg.bt = pg.bt + b0 * pg.max_blocks;
    kp.table = nullptr;
    kp.krot = base + p.krot + b0 * ws_seq;
    kp.vt = dtype == DCA_BF16 ? base + p.vt + b0 * ws_seq : nullptr;
    kp.B = nb;
    kp.in_rows = (int)cache_len;
    kp.Lp = (int)p.Lp;
    kp.Hkv = (int)Hkv;
    kp.D = (int)D;
    kp.kdiv = 1;
    kp.kmod = 1 << 30;
    kp.per_seq = 1;
    PrefillArgs a = {};
    for (int i = 0; i < nb; ++i) {
      const int64_t n = q_len ? q_len[b0 + i] : Lq;
      kp.seq_len[i] = (int)(pos0[b0 + i] + n);
      a.seq_q0[i] = (int)pos0[b0 + i];
      a.seq_len[i] = (int)n;
    }
    kp.L = (int)max_keys;
    if (launch_kv_prep(kp, dtype, st) != hipSuccess) return DCA_ERR_HIP;
    a.q = (const uint8_t*)q + b0 * Lq * Hq * D * es;
    a.krot = kp.krot;
    a.krot2 = nullptr;
    // bf16 reads the V tiles; fp32 reads the cache's values directly
    a.vt = dtype == DCA_BF16 ? kp.vt : kp.v;
    if (dtype == DCA_BF16)
      a.ftable = (const float2*)table;
    else
      a.table = table;
    a.tab_ps = 1;   // frequency-major
    a.tab_ks = c;
    a.o = (uint8_t*)o + b0 * Lq * Hq * D * es;
    a.lse = lse ? lse + b0 * Hq * Lq : nullptr;
    a.B = nb;
    a.L = (int)max_keys;
    a.Lp = (int)p.Lp;
    a.Hq = (int)Hq;
    a.Hkv = (int)Hkv;
    a.D = (int)D;
    a.c = c;
    a.w = w;
    a.s = c - w;
    a.map = kMapDCA;
    a.se_group = 1;
    a.q_rows = (int)Lq;
    a.per_seq = 1;
    a.v_rows = (int)cache_len;
    a.pg = kp.pg;
    a.sm_scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)D));
    const hipError_t e = dtype == DCA_BF16 ? launch_prefill_bf16(a, st) : launch_prefill_f32(a, st);
    if (e != hipSuccess) return DCA_ERR_HIP;
  }
  return DCA_OK;
}

// Decode with per-sequence cache lengths over a dense cache (pg.bt null) or a
// paged one (cache_len = the most rows a sequence's table covers).
// The position map of a decode call.  SelfExtend and coarse / fine read the
// keys below a per-sequence boundary from a second cache (kc2).
struct DecodeMap {
  int map = kMapDCA;
  const void* kc2 = nullptr;
  int se_group = 1, se_window = 0;
  int cf_chunk = 1;
  double cf_inv_kappa = 1.0;
};

// First key read from the main cache: SelfExtend, the first neighbor key of
// the new token kv - 1 (j > kv - 1 - W); coarse / fine, the first key of the
// chunk before the new token's chunk; DCA: 0.
int64_t map_seg(const DecodeMap& m, int64_t kv) {
  if (m.map == kMapSelfExtend) return kv - m.se_window > 0 ? kv - m.se_window : 0;
  if (m.map == kMapCoarseFine) {
    const int64_t ci = (kv - 1) / m.cf_chunk;
    return ci >= 1 ? (ci - 1) * m.cf_chunk : 0;
  }
  return 0;
}

// Workspace layout of a ragged decode under a map, and each sequence's first
// key read from the main cache (two-cache maps).
bool map_decode_layout(const int64_t* kv_len, int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int dtype,
                       const DecodeMap& m, DecodeLayout* p, std::vector<int64_t>* seg_out) {
  if (!kv_len || B < 1 || B >= kMaxDim) return false;
  int64_t max_kv = 0;
  std::vector<int64_t> seg(m.map == kMapDCA ? 0 : (size_t)B);
  for (int64_t b = 0; b < B; ++b) {
    if (kv_len[b] < 1 || kv_len[b] >= kMaxDim / 2) return false;
    max_kv = kv_len[b] > max_kv ? kv_len[b] : max_kv;
    if (m.map != kMapDCA) seg[b] = map_seg(m, kv_len[b]);
  }
  if (!decode_layout(B, kv_len, max_kv, Hq, Hkv, D, dtype, p)) return false;
  if (seg_out) *seg_out = seg;
  return true;
}

int decode_varlen_impl(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                       const int64_t* kv_len, int64_t B, int64_t cache_len, int64_t Hq, int64_t Hkv,
                       int64_t D, int c, int w, double rope_base, float sm_scale, int dtype, void* ws,
                       size_t ws_bytes, void* stream, const PagedKv& pg, const DecodeMap& dm = DecodeMap{},
                       size_t* need_bytes = nullptr) {
  // need_bytes non-null: validate every argument, store the scratch bytes the
  // call needs and return without touching the device.
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !o || !kv_len) return DCA_ERR_INVALID_ARG;
  if (B < 1 || cache_len < 1 || cache_len >= kMaxDim / 2 || Hq < 1 || Hkv < 1 || Hq % Hkv)
    return DCA_ERR_INVALID_ARG;
  if ((dm.map == kMapDCA && !cw_ok(c, w)) || !base_ok(rope_base) || !isfinite(sm_scale)) return DCA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return DCA_ERR_INVALID_ARG;
  if (dm.map != kMapDCA && (!dm.kc2 || !aligned(dm.kc2, 16))) return DCA_ERR_INVALID_ARG;
  int64_t max_kv = 0;
  for (int64_t b = 0; b < B; ++b) {
    if (kv_len[b] < 1 || kv_len[b] > cache_len) return DCA_ERR_INVALID_ARG;
    max_kv = kv_len[b] > max_kv ? kv_len[b] : max_kv;
  }
  DecodeLayout p;
  std::vector<int64_t> seg;
  if (!map_decode_layout(kv_len, B, Hq, Hkv, D, dtype, dm, &p, &seg)) return DCA_ERR_INVALID_ARG;
  if (need_bytes) {
    *need_bytes = p.total;
    return DCA_OK;
  }
  if (!ws || ws_bytes < p.total || !aligned(ws, 256)) return DCA_ERR_WORKSPACE;
  uint8_t* base = (uint8_t*)ws;
  const int64_t es = elem_size(dtype);
  for (int64_t b0 = 0; b0 < B; b0 += kMaxSeqGroup) {
    const int nb = (int)(B - b0 < kMaxSeqGroup ? B - b0 : kMaxSeqGroup);
    DecodeArgs a = {};
    a.q = (const uint8_t*)q + b0 * Hq * D * es;
    a.kc = (const uint8_t*)k_cache + (pg.bt ? 0 : b0 * cache_len * Hkv * D * es);
    a.vc = (const uint8_t*)v_cache + (pg.bt ? 0 : b0 * cache_len * Hkv * D * es);
    a.pg = pg;
    if (pg.bt) a.pg.bt = pg.bt + b0 * pg.max_blocks;
    a.o = (uint8_t*)o + b0 * Hq * D * es;
    a.lse = lse ? lse + b0 * Hq : nullptr;
    a.qv = base + p.qv + b0 * Hq * 3 * D * es;
    a.part_o = (float*)(base + p.part_o) + b0 * Hq * (int64_t)p.ns * D;
    a.part_lse = (float*)(base + p.part_lse) + b0 * Hq * (int64_t)p.ns;
    a.B = nb;
    a.kv_len = (int)max_kv;
    a.Hq = (int)Hq;
    a.Hkv = (int)Hkv;
    a.D = (int)D;
    a.c = c;
    a.w = w;
    a.s = c - w;
    a.base = rope_base;
    a.sm_scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)D));
    a.keys_per_split = p.kps;
    a.nsplit = p.ns;
    a.cache_len = (int)cache_len;
    a.per_seq = 1;
    for (int i = 0; i < nb; ++i) a.seq_len[i] = (int)kv_len[b0 + i];
    a.map = dm.map;
    if (dm.map != kMapDCA) {
      a.kc2 = (const uint8_t*)dm.kc2 + (pg.bt ? 0 : b0 * cache_len * Hkv * D * es);
      for (int i = 0; i < nb; ++i) a.seg[i] = (int)seg[b0 + i];
    }
    a.se_group = dm.se_group;
    a.se_window = dm.se_window;
    a.cf_inv_kappa = dm.cf_inv_kappa;
    const hipError_t e = launch_decode(a, dtype, (hipStream_t)stream);
    if (e != hipSuccess) return DCA_ERR_HIP;
  }
  return DCA_OK;
}

// Paged-cache arguments: pool sizes and the block table (device memory, not
// read on the host).  page_size must be a multiple of 16.
bool paged_ok(const int32_t* block_table, int64_t B, int64_t num_pages, int64_t page_size, int64_t max_blocks,
              PagedKv* pg) {
  if (!block_table || !aligned(block_table, 4)) return false;
  if (num_pages < 1 || num_pages >= kMaxDim || page_size < 16 || page_size % 16 || page_size >= kMaxDim / 2)
    return false;
  if (max_blocks < 1 || max_blocks >= kMaxDim || B * max_blocks >= kMaxDim) return false;
  if (max_blocks * page_size >= kMaxDim / 2) return false;
  pg->bt = block_table;
  pg->page_size = (int)page_size;
  pg->max_blocks = (int)max_blocks;
  pg->num_pages = (int)num_pages;
  return true;
}

// ---- scratch for the entry point that allocates nothing ------------------------
// dca_decode_paged_noalloc keeps the decode's partial results (rotated query
// variants, per-range O and LSE) in this file-scope device array instead of a
// caller workspace.  Each GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code `scratch` names only a
// host-side stand-in, so kernels are handed the device address that
// hipGetSymbolAddress returns, taken once per device (with that device
// current) and kept here.
constexpr size_t kScratchBytes = DCA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxScratchDevices];

// Device address of the current device's scratch array (set up on the first
// call on that device).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return DCA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DCA_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return DCA_OK;
}

}  // namespace

extern "C" {

size_t dca_decode_varlen_workspace_bytes(const int64_t* kv_len, int64_t B, int64_t Hq, int64_t Hkv,
                                         int64_t D, int dtype) {
  DecodeLayout p;
  return map_decode_layout(kv_len, B, Hq, Hkv, D, dtype, DecodeMap{}, &p, nullptr) ? p.total : 0;
}

int dca_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int64_t* pos0, const int64_t* q_len, int64_t B, int64_t Lq, int64_t cache_len,
                      int64_t Hq, int64_t Hkv, int64_t D, int c, int w, double rope_base, float sm_scale,
                      int dtype, void* ws, size_t ws_bytes, void* stream) {
  return prefill_chunk_impl(q, k_cache, v_cache, o, lse, pos0, q_len, B, Lq, cache_len, Hq, Hkv, D, c, w,
                            rope_base, sm_scale, dtype, ws, ws_bytes, stream, PagedKv{});
}

int dca_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int64_t* kv_len, int64_t B, int64_t cache_len, int64_t Hq, int64_t Hkv,
                      int64_t D, int c, int w, double rope_base, float sm_scale, int dtype, void* ws,
                      size_t ws_bytes, void* stream) {
  return decode_varlen_impl(q, k_cache, v_cache, o, lse, kv_len, B, cache_len, Hq, Hkv, D, c, w, rope_base,
                            sm_scale, dtype, ws, ws_bytes, stream, PagedKv{});
}

int dca_prefill_chunk_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                            void* o, float* lse, const int64_t* pos0, const int64_t* q_len, int64_t B, int64_t Lq,
                            int64_t num_pages, int64_t page_size, int64_t max_blocks, int64_t Hq, int64_t Hkv,
                            int64_t D, int c, int w, double rope_base, float sm_scale, int dtype, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  PagedKv pg;
  if (!paged_ok(block_table, B, num_pages, page_size, max_blocks, &pg)) return DCA_ERR_INVALID_ARG;
  return prefill_chunk_impl(q, k_pages, v_pages, o, lse, pos0, q_len, B, Lq, max_blocks * page_size, Hq, Hkv,
                            D, c, w, rope_base, sm_scale, dtype, ws, ws_bytes, stream, pg);
}

int dca_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table, void* o,
                     float* lse, const int64_t* kv_len, int64_t B, int64_t num_pages, int64_t page_size,
                     int64_t max_blocks, int64_t Hq, int64_t Hkv, int64_t D, int c, int w, double rope_base,
                     float sm_scale, int dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  PagedKv pg;
  if (!paged_ok(block_table, B, num_pages, page_size, max_blocks, &pg)) return DCA_ERR_INVALID_ARG;
  return decode_varlen_impl(q, k_pages, v_pages, o, lse, kv_len, B, max_blocks * page_size, Hq, Hkv, D, c, w,
                            rope_base, sm_scale, dtype, ws, ws_bytes, stream, pg);
}

int dca_decode_paged_noalloc(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                             void* o, float* lse, const int64_t* kv_len, int64_t B, int64_t num_pages,
                             int64_t page_size, int64_t max_blocks, int64_t Hq, int64_t Hkv, int64_t D, int c, int w,
                             double rope_base, float sm_scale, int dtype, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  PagedKv pg;
  if (!paged_ok(block_table, B, num_pages, page_size, max_blocks, &pg)) return DCA_ERR_INVALID_ARG;
  // Every argument is checked, and the scratch the call needs sized, before
  // the first HIP call.
  size_t need = 0;
  const int64_t cache_len = max_blocks * page_size;
  int r = decode_varlen_impl(q, k_pages, v_pages, o, lse, kv_len, B, cache_len, Hq, Hkv, D, c, w, rope_base,
                             sm_scale, dtype, nullptr, 0, stream, pg, DecodeMap{}, &need);
  if (r != DCA_OK) return r;
  if (need > kScratchBytes) return DCA_ERR_TOO_LARGE;
  void* ws = nullptr;
  r = scratch_address(&ws);
  if (r != DCA_OK) return r;
  // The kernels write every partial they later read (no part of the scratch
  // has to start at zero).
  return decode_varlen_impl(q, k_pages, v_pages, o, lse, kv_len, B, cache_len, Hq, Hkv, D, c, w, rope_base,
                            sm_scale, dtype, ws, kScratchBytes, stream, pg);
}


size_t dca_selfextend_decode_workspace_bytes(const int64_t* kv_len, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                             int group, int window, int dtype) {
  if (!se_ok(group, window)) return 0;
  DecodeMap m;
  m.map = kMapSelfExtend;
  m.se_group = group;
  m.se_window = window;
  DecodeLayout p;
  return map_decode_layout(kv_len, B, Hq, Hkv, D, dtype, m, &p, nullptr) ? p.total : 0;
}

int dca_selfextend_decode(const void* q, const void* k_cache, const void* k_cache_grouped, const void* v_cache,
                          void* o, float* lse, const int64_t* kv_len, int64_t B, int64_t cache_len, int64_t Hq,
                          int64_t Hkv, int64_t D, int group, int window, double rope_base, float sm_scale,
                          int dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!se_ok(group, window) || !k_cache_grouped) return DCA_ERR_INVALID_ARG;
  DecodeMap m;
  m.map = kMapSelfExtend;
  m.kc2 = k_cache_grouped;
  m.se_group = group;
  m.se_window = window;
  const int unbounded = 1 << 30;   // no chunk relation: s never splits a range
  return decode_varlen_impl(q, k_cache, v_cache, o, lse, kv_len, B, cache_len, Hq, Hkv, D, unbounded, 0,
                            rope_base, sm_scale, dtype, ws, ws_bytes, stream, PagedKv{}, m);
}

size_t dca_coarse_fine_decode_workspace_bytes(const int64_t* kv_len, int64_t B, int64_t Hq, int64_t Hkv,
                                              int64_t D, int chunk, int dtype) {
  if (chunk < 1 || chunk > (1 << 24)) return 0;
  DecodeMap m;
  m.map = kMapCoarseFine;
  m.cf_chunk = chunk;
  DecodeLayout p;
  return map_decode_layout(kv_len, B, Hq, Hkv, D, dtype, m, &p, nullptr) ? p.total : 0;
}

int dca_coarse_fine_decode(const void* q, const void* k_cache, const void* k_cache_scaled, const void* v_cache,
                           void* o, float* lse, const int64_t* kv_len, int64_t B, int64_t cache_len, int64_t Hq,
                           int64_t Hkv, int64_t D, int chunk, int train_len, int target_len, double rope_base,
                           float sm_scale, int dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (chunk < 1 || chunk > (1 << 24) || train_len < 1 || target_len < 1 || !k_cache_scaled)
    return DCA_ERR_INVALID_ARG;
  DecodeMap m;
  m.map = kMapCoarseFine;
  m.kc2 = k_cache_scaled;
  m.cf_chunk = chunk;
  m.cf_inv_kappa = (double)train_len / (double)target_len;
  // the chunk relation uses chunk size C (held in c and s)
  return decode_varlen_impl(q, k_cache, v_cache, o, lse, kv_len, B, cache_len, Hq, Hkv, D, chunk, 0, rope_base,
                            sm_scale, dtype, ws, ws_bytes, stream, PagedKv{}, m);
}

// The two-cache map decodes over page pools: both key pools and the value
// pool share one block table.
int dca_selfextend_decode_paged(const void* q, const void* k_pages, const void* k_pages_2nd, const void* v_pages,
                                const int32_t* block_table, void* o, float* lse, const int64_t* kv_len, int64_t B,
                                int64_t num_pages, int64_t page_size, int64_t max_blocks, int64_t Hq, int64_t Hkv,
                                int64_t D, int group, int window, double rope_base, float sm_scale, int dtype,
                                void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!se_ok(group, window) || !k_pages_2nd) return DCA_ERR_INVALID_ARG;
  PagedKv pg;
  if (!paged_ok(block_table, B, num_pages, page_size, max_blocks, &pg)) return DCA_ERR_INVALID_ARG;
  DecodeMap m;
  m.map = kMapSelfExtend;
  m.kc2 = k_pages_2nd;
  m.se_group = group;
  m.se_window = window;
  const int unbounded = 1 << 30;   // no chunk relation: s never splits a range
  return decode_varlen_impl(q, k_pages, v_pages, o, lse, kv_len, B, max_blocks * page_size, Hq, Hkv, D, unbounded,
                            0, rope_base, sm_scale, dtype, ws, ws_bytes, stream, pg, m);
}

int dca_coarse_fine_decode_paged(const void* q, const void* k_pages, const void* k_pages_2nd, const void* v_pages,
                                 const int32_t* block_table, void* o, float* lse, const int64_t* kv_len, int64_t B,
                                 int64_t num_pages, int64_t page_size, int64_t max_blocks, int64_t Hq, int64_t Hkv,
                                 int64_t D, int chunk, int train_len, int target_len, double rope_base,
                                 float sm_scale, int dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (chunk < 1 || chunk > (1 << 24) || train_len < 1 || target_len < 1 || !k_pages_2nd)
    return DCA_ERR_INVALID_ARG;
  PagedKv pg;
  if (!paged_ok(block_table, B, num_pages, page_size, max_blocks, &pg)) return DCA_ERR_INVALID_ARG;
  DecodeMap m;
  m.map = kMapCoarseFine;
  m.kc2 = k_pages_2nd;
  m.cf_chunk = chunk;
  m.cf_inv_kappa = (double)train_len / (double)target_len;
  return decode_varlen_impl(q, k_pages, v_pages, o, lse, kv_len, B, max_blocks * page_size, Hq, Hkv, D, chunk, 0,
                            rope_base, sm_scale, dtype, ws, ws_bytes, stream, pg, m);
}

int dca_coarse_fine_key_remap(const void* x, void* out, int64_t B, int64_t L, int64_t H, int64_t D, int64_t pos0,
                              int chunk, int train_len, int target_len, double rope_base, int dtype, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(D)) return DCA_ERR_UNSUPPORTED;
  if (!x || !out || B < 0 || L < 0 || H < 0 || pos0 < 0) return DCA_ERR_INVALID_ARG;
  if (B >= kMaxDim || L >= kMaxDim || H * D >= kMaxDim || pos0 > (int64_t(1) << 52)) return DCA_ERR_INVALID_ARG;
  if (chunk < 1 || chunk > (1 << 24) || train_len < 1 || target_len < 1 || !base_ok(rope_base))
    return DCA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(out, 16)) return DCA_ERR_INVALID_ARG;
  if (B == 0 || L == 0 || H == 0) return DCA_OK;
  const double step = (double)chunk * (double)train_len / (double)target_len;
  return hip_status(launch_rope_remap(x, out, B, L, H, D, pos0, kRemapCoarseScaled, chunk, 0, rope_base, dtype,
                                      (hipStream_t)stream, step));
}

}  // extern "C"
