"""MI355X (gfx950) Dual Chunk Attention: thin Python binding of the C ABI.

Every step of the computation runs in the HIP kernels of ``libdca_mi355x.so``;
this module only checks tensors, allocates outputs/workspaces through PyTorch
(device memory and the current stream are all PyTorch supplies) and passes
pointers.  There is no CPU fallback: if the library is missing, every entry
point raises.

Entry points (same names as include/dca.h):
  rope_remap(x, map, c, w, base=1e4, pos0=0, out=None)
  prefill(q, k, v, c, w, base=1e4, sm_scale=None, return_lse=False,
          return_k_rot=False, workspace=None)
  decode(q, k_cache, v_cache, c, w, base=1e4, sm_scale=None,
         return_lse=False, workspace=None)
  selfextend_prefill(q, k, v, group, window, base=1e4, sm_scale=None,
                     return_lse=False, workspace=None)
  coarse_fine_prefill(q, k, v, chunk, train_len, target_len, base=1e4,
                      sm_scale=None, return_lse=False, workspace=None)
  prefill_chunk(q, k_cache, v_cache, pos0, c, w, base=1e4, sm_scale=None,
                q_len=None, return_lse=False, out=None, workspace=None)
  decode_varlen(q, k_cache, v_cache, kv_len, c, w, base=1e4, sm_scale=None,
                return_lse=False, workspace=None)
  prefill_workspace_bytes(...), decode_workspace_bytes(...),
  selfextend_workspace_bytes(...)
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (  # noqa: F401
    DCA_BF16, DCA_F32, DCA_MAP_KEY, DCA_MAP_PLAIN, DCA_MAP_Q_INTER, DCA_MAP_Q_INTRA,
    DCA_MAP_Q_SUCC, DCA_MAP_SE_KEY_GROUPED, DCA_MAP_SE_Q_GROUPED, DCA_NOALLOC_SCRATCH_BYTES, DCAError,
)

__all__ = ["rope_remap", "prefill", "prefill_prepare", "prefill_attend", "decode",
           "selfextend_prefill", "prefill_chunk", "decode_varlen", "decode_paged", "decode_paged_noalloc", "prefill_chunk_paged",
           "coarse_fine_prefill", "selfextend_decode", "coarse_fine_decode", "selfextend_decode_paged",
           "coarse_fine_decode_paged", "coarse_fine_key_remap", "prefill_workspace_bytes", "decode_workspace_bytes",
           "selfextend_workspace_bytes", "decode_varlen_workspace_bytes", "coarse_fine_workspace_bytes",
           "selfextend_decode_workspace_bytes", "coarse_fine_decode_workspace_bytes", "DCAError", "library_path"]

_DT = {torch.float32: DCA_F32, torch.bfloat16: DCA_BF16}


def library_path() -> str:
    return _lib.LIB_PATH


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"dtype {t.dtype} not supported (float32 or bfloat16)")
    return _DT[t.dtype]


def _check(t: torch.Tensor, name: str, ndim: int, dtype=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_out(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    """A caller-supplied output: the kernels write exactly `shape` elements of
    `dtype` on `device`, densely, so anything else is refused before the call
    (a smaller buffer would be written past its end)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def prefill_workspace_bytes(B, L, Hkv, D, c, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    return int(_lib.load().dca_prefill_workspace_bytes(B, L, Hkv, D, c, code))


def decode_workspace_bytes(B, kv_len, Hq, Hkv, D, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    return int(_lib.load().dca_decode_workspace_bytes(B, kv_len, Hq, Hkv, D, code))


def selfextend_workspace_bytes(B, L, Hkv, D, group, window, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    return int(_lib.load().dca_selfextend_workspace_bytes(B, L, Hkv, D, group, window, code))


def coarse_fine_workspace_bytes(B, L, Hkv, D, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    return int(_lib.load().dca_coarse_fine_workspace_bytes(B, L, Hkv, D, code))


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if (not isinstance(workspace, torch.Tensor) or workspace.device != torch.device(device)
            or not workspace.is_contiguous() or workspace.numel() * workspace.element_size() < nbytes):
        raise ValueError(f"workspace must be a contiguous buffer of at least {nbytes} bytes on {device}")
    return workspace


def rope_remap(x: torch.Tensor, map: int, c: int, w: int, base: float = 10000.0, pos0: int = 0,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """Rotate x [B, L, H, D] by position map `map` (token t at pos0 + t).  For the
    SelfExtend grouped maps, c is the group size and w the window."""
    lib = _lib.load()
    _check(x, "x", 4)
    if out is None:
        out = torch.empty_like(x)
    _check_out(out, "out", x.shape, x.dtype, x.device)
    B, L, H, D = x.shape
    _lib.check("dca_rope_remap", lib.dca_rope_remap(
        x.data_ptr(), out.data_ptr(), B, L, H, D, pos0, map, c, w, float(base), _dtype_code(x),
        _stream(x.device)))
    return out


def prefill(q, k, v, c: int, w: int, base: float = 10000.0, sm_scale: float | None = None,
            return_lse: bool = False, return_k_rot: bool = False, workspace=None):
    """DCA causal prefill.  q [B, L, Hq, D], k/v [B, L, Hkv, D] raw; returns o (and lse, k_rot)."""
    lib = _lib.load()
    _check(q, "q", 4)
    _check(k, "k", 4, q.dtype)
    _check(v, "v", 4, q.dtype)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, L, Hkv, D) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    code = _dtype_code(q)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, L, dtype=torch.float32, device=q.device) if return_lse else None
    k_rot = torch.empty_like(k) if return_k_rot else None
    nbytes = int(lib.dca_prefill_workspace_bytes(B, L, Hkv, D, c, code))
    if nbytes == 0:
        raise ValueError("invalid prefill sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check("dca_prefill", lib.dca_prefill(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse), _ptr(k_rot),
        B, L, Hq, Hkv, D, c, w, float(base), float(sm_scale or 0.0), code,
        ws.data_ptr(), nbytes, _stream(q.device)))
    res = [o]
    if return_lse:
        res.append(lse)
    if return_k_rot:
        res.append(k_rot)
    return res[0] if len(res) == 1 else tuple(res)


def prefill_prepare(k, v, c: int, w: int, base: float = 10000.0, workspace=None,
                    k_rot_out: torch.Tensor | None = None) -> torch.Tensor:
    """Phase 1 of prefill: build the rotated-key / value workspace; returns it."""
    lib = _lib.load()
    _check(k, "k", 4)
    _check(v, "v", 4, k.dtype)
    B, L, Hkv, D = k.shape
    code = _dtype_code(k)
    nbytes = int(lib.dca_prefill_workspace_bytes(B, L, Hkv, D, c, code))
    if nbytes == 0:
        raise ValueError("invalid prefill sizes")
    ws = _workspace(nbytes, k.device, workspace)
    if k_rot_out is not None:
        _check_out(k_rot_out, "k_rot_out", k.shape, k.dtype, k.device)
    _lib.check("dca_prefill_prepare", lib.dca_prefill_prepare(
        k.data_ptr(), v.data_ptr(), _ptr(k_rot_out), B, L, Hkv, D, c, w, float(base), code,
        ws.data_ptr(), nbytes, _stream(k.device)))
    return ws


def prefill_attend(q, workspace, Hkv: int, c: int, w: int, sm_scale: float | None = None,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Phase 2 of prefill: the attention kernel over a prepared workspace."""
    lib = _lib.load()
    _check(q, "q", 4)
    B, L, Hq, D = q.shape
    code = _dtype_code(q)
    o = torch.empty_like(q) if out is None else out
    _check_out(o, "out", q.shape, q.dtype, q.device)
    if lse is not None:
        _check_out(lse, "lse", (B, Hq, L), torch.float32, q.device)
    nbytes = int(lib.dca_prefill_workspace_bytes(B, L, Hkv, D, c, code))
    if nbytes == 0:
        raise ValueError("invalid prefill sizes")
    if workspace.device != q.device or workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a buffer of at least {nbytes} bytes on {q.device}")
    _lib.check("dca_prefill_attend", lib.dca_prefill_attend(
        q.data_ptr(), o.data_ptr(), _ptr(lse), B, L, Hq, Hkv, D, c, w, float(sm_scale or 0.0), code,
        workspace.data_ptr(), nbytes, _stream(q.device)))
    return o


def decode(q, k_cache, v_cache, c: int, w: int, base: float = 10000.0, sm_scale: float | None = None,
           return_lse: bool = False, workspace=None):
    """DCA decode of one token per sequence: q [B, Hq, D] raw; caches [B, kv_len, Hkv, D],
    keys already rotated at j mod s.  The token sits at position kv_len - 1."""
    lib = _lib.load()
    _check(q, "q", 3)
    _check(k_cache, "k_cache", 4, q.dtype)
    _check(v_cache, "v_cache", 4, q.dtype)
    B, Hq, D = q.shape
    kv_len, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, kv_len, Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    code = _dtype_code(q)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = int(lib.dca_decode_workspace_bytes(B, kv_len, Hq, Hkv, D, code))
    if nbytes == 0:
        raise ValueError("invalid decode sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check("dca_decode", lib.dca_decode(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), _ptr(lse),
        B, kv_len, Hq, Hkv, D, c, w, float(base), float(sm_scale or 0.0), code,
        ws.data_ptr(), nbytes, _stream(q.device)))
    return (o, lse) if return_lse else o


def selfextend_prefill(q, k, v, group: int, window: int, base: float = 10000.0,
                       sm_scale: float | None = None, return_lse: bool = False, workspace=None):
    """SelfExtend grouped / neighbor causal prefill.  q [B, L, Hq, D], k/v [B, L, Hkv, D] raw;
    returns o (and lse)."""
    lib = _lib.load()
    _check(q, "q", 4)
    _check(k, "k", 4, q.dtype)
    _check(v, "v", 4, q.dtype)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, L, Hkv, D) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    code = _dtype_code(q)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, L, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = int(lib.dca_selfextend_workspace_bytes(B, L, Hkv, D, group, window, code))
    if nbytes == 0:
        raise ValueError("invalid SelfExtend prefill sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check("dca_selfextend_prefill", lib.dca_selfextend_prefill(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse),
        B, L, Hq, Hkv, D, group, window, float(base), float(sm_scale or 0.0), code,
        ws.data_ptr(), nbytes, _stream(q.device)))
    return (o, lse) if return_lse else o


def _host_i64(values, n: int, name: str):
    """A host int64 array of n entries for the C ABI (an int broadcasts)."""
    if isinstance(values, int):
        values = [values] * n
    values = [int(x) for x in (values.tolist() if hasattr(values, "tolist") else values)]
    if len(values) != n:
        raise ValueError(f"{name} needs {n} entries, got {len(values)}")
    return (ctypes.c_int64 * n)(*values), values


def prefill_chunk(q, k_cache, v_cache, pos0, c: int, w: int, base: float = 10000.0,
                  sm_scale: float | None = None, q_len=None, return_lse: bool = False, out=None,
                  workspace=None):
    """Chunked DCA prefill over a KV cache.  q [B, Lq, Hq, D] raw queries of the new
    tokens (row r of sequence b at position pos0[b] + r); caches [B, cache_len, Hkv, D]
    with keys already rotated at j mod s, the chunk's own keys included.  pos0 and
    q_len: an int or one entry per sequence (q_len None: Lq rows each).  Rows past
    q_len[b] of the output are left as they were (zeros when out is None)."""
    lib = _lib.load()
    _check(q, "q", 4)
    _check(k_cache, "k_cache", 4, q.dtype)
    _check(v_cache, "v_cache", 4, q.dtype)
    B, Lq, Hq, D = q.shape
    cache_len, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, cache_len, Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    code = _dtype_code(q)
    p0, p0v = _host_i64(pos0, B, "pos0")
    if q_len is None:
        ql, qlv = None, [Lq] * B
    else:
        ql, qlv = _host_i64(q_len, B, "q_len")
    o = torch.zeros_like(q) if out is None else out
    _check_out(o, "out", q.shape, q.dtype, q.device)
    lse = torch.full((B, Hq, Lq), float("-inf"), dtype=torch.float32, device=q.device) if return_lse else None
    max_keys = max(a + n for a, n in zip(p0v, qlv))
    nbytes = int(lib.dca_prefill_workspace_bytes(B, max(max_keys, 1), Hkv, D, c, code))
    if nbytes == 0:
        raise ValueError("invalid chunked prefill sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check("dca_prefill_chunk", lib.dca_prefill_chunk(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), _ptr(lse), p0, ql,
        B, Lq, cache_len, Hq, Hkv, D, c, w, float(base), float(sm_scale or 0.0), code,
        ws.data_ptr(), nbytes, _stream(q.device)))
    return (o, lse) if return_lse else o


def decode_varlen_workspace_bytes(kv_len, Hq, Hkv, D, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    n = len(kv_len) if not isinstance(kv_len, int) else 1
    kl, _ = _host_i64(kv_len, n, "kv_len")
    return int(_lib.load().dca_decode_varlen_workspace_bytes(kl, n, Hq, Hkv, D, code))


def decode_varlen(q, k_cache, v_cache, kv_len, c: int, w: int, base: float = 10000.0,
                  sm_scale: float | None = None, return_lse: bool = False, workspace=None):
    """DCA decode of a ragged batch: sequence b holds kv_len[b] cached tokens (its new
    token at kv_len[b] - 1).  q [B, Hq, D] raw; caches [B, cache_len, Hkv, D], keys
    rotated at j mod s."""
    lib = _lib.load()
    _check(q, "q", 3)
    _check(k_cache, "k_cache", 4, q.dtype)
    _check(v_cache, "v_cache", 4, q.dtype)
    B, Hq, D = q.shape
    cache_len, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, cache_len, Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    code = _dtype_code(q)
    kl, klv = _host_i64(kv_len, B, "kv_len")
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = int(lib.dca_decode_varlen_workspace_bytes(kl, B, Hq, Hkv, D, code))
    if nbytes == 0:
        raise ValueError("invalid decode sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check("dca_decode_varlen", lib.dca_decode_varlen(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), _ptr(lse), kl,
        B, cache_len, Hq, Hkv, D, c, w, float(base), float(sm_scale or 0.0), code,
        ws.data_ptr(), nbytes, _stream(q.device)))
    return (o, lse) if return_lse else o


def _check_pages(k_pages, v_pages, block_table, q):
    _check(k_pages, "k_pages", 4, q.dtype)
    _check(v_pages, "v_pages", 4, q.dtype)
    if v_pages.shape != k_pages.shape:
        raise ValueError("k_pages and v_pages differ in shape")
    if (block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous()
            or block_table.device != q.device):
        raise ValueError("block_table must be a contiguous int32 [B, max_blocks] tensor on q's device")
    return k_pages.shape[0], k_pages.shape[1], k_pages.shape[2], block_table.shape[1]


def decode_paged(q, k_pages, v_pages, block_table, kv_len, c: int, w: int, base: float = 10000.0,
                 sm_scale: float | None = None, return_lse: bool = False, workspace=None):
    """DCA decode over a paged cache: pools [num_pages, page_size, Hkv, D] (keys rotated
    at j mod s), block_table int32 [B, max_blocks] on the device (row j of sequence b
    at row j % page_size of page block_table[b, j // page_size]), kv_len per sequence.
    page_size must be a multiple of 16."""
    lib = _lib.load()
    _check(q, "q", 3)
    num_pages, page_size, Hkv, max_blocks = _check_pages(k_pages, v_pages, block_table, q)
    B, Hq, D = q.shape
    if k_pages.shape[3] != D or block_table.shape[0] != B:
        raise ValueError("page pool / block table shapes do not match q")
    code = _dtype_code(q)
    kl, _ = _host_i64(kv_len, B, "kv_len")
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = int(lib.dca_decode_varlen_workspace_bytes(kl, B, Hq, Hkv, D, code))
    if nbytes == 0:
        raise ValueError("invalid decode sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check("dca_decode_paged", lib.dca_decode_paged(
        q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(), o.data_ptr(), _ptr(lse),
        kl, B, num_pages, page_size, max_blocks, Hq, Hkv, D, c, w, float(base), float(sm_scale or 0.0), code,
        ws.data_ptr(), nbytes, _stream(q.device)))
    return (o, lse) if return_lse else o


def decode_paged_noalloc(q, k_pages, v_pages, block_table, kv_len, c: int, w: int, base: float = 10000.0,
                         sm_scale: float | None = None, out=None, lse=None):
    """decode_paged without a workspace: the library keeps the decode's scratch in a
    static device buffer of DCA_NOALLOC_SCRATCH_BYTES per GPU (calls that overlap on
    one GPU race on it).  Pass `out` (and `lse`) to make the call allocate nothing;
    they are allocated here when None.  Returns out (and lse when given)."""
    lib = _lib.load()
    _check(q, "q", 3)
    num_pages, page_size, Hkv, max_blocks = _check_pages(k_pages, v_pages, block_table, q)
    B, Hq, D = q.shape
    if k_pages.shape[3] != D or block_table.shape[0] != B:
        raise ValueError("page pool / block table shapes do not match q")
    code = _dtype_code(q)
    kl, _ = _host_i64(kv_len, B, "kv_len")
    o = torch.empty_like(q) if out is None else out
    _check_out(o, "out", q.shape, q.dtype, q.device)
    if lse is not None:
        _check_out(lse, "lse", (B, Hq), torch.float32, q.device)
    with torch.cuda.device(q.device):   # the scratch used is the current device's
        _lib.check("dca_decode_paged_noalloc", lib.dca_decode_paged_noalloc(
            q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(), o.data_ptr(),
            _ptr(lse), kl, B, num_pages, page_size, max_blocks, Hq, Hkv, D, c, w, float(base),
            float(sm_scale or 0.0), code, _stream(q.device)))
    return o if lse is None else (o, lse)


def prefill_chunk_paged(q, k_pages, v_pages, block_table, pos0, c: int, w: int, base: float = 10000.0,
                        sm_scale: float | None = None, q_len=None, return_lse: bool = False, out=None,
                        workspace=None):
    """Chunked DCA prefill over a paged cache (layout as in decode_paged); otherwise as
    prefill_chunk."""
    lib = _lib.load()
    _check(q, "q", 4)
    num_pages, page_size, Hkv, max_blocks = _check_pages(k_pages, v_pages, block_table, q)
    B, Lq, Hq, D = q.shape
    if k_pages.shape[3] != D or block_table.shape[0] != B:
        raise ValueError("page pool / block table shapes do not match q")
    code = _dtype_code(q)
    p0, p0v = _host_i64(pos0, B, "pos0")
    if q_len is None:
        ql, qlv = None, [Lq] * B
    else:
        ql, qlv = _host_i64(q_len, B, "q_len")
    o = torch.zeros_like(q) if out is None else out
    _check_out(o, "out", q.shape, q.dtype, q.device)
    lse = torch.full((B, Hq, Lq), float("-inf"), dtype=torch.float32, device=q.device) if return_lse else None
    max_keys = max(a + n for a, n in zip(p0v, qlv))
    nbytes = int(lib.dca_prefill_workspace_bytes(B, max(max_keys, 1), Hkv, D, c, code))
    if nbytes == 0:
        raise ValueError("invalid chunked prefill sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check("dca_prefill_chunk_paged", lib.dca_prefill_chunk_paged(
        q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(), o.data_ptr(), _ptr(lse),
        p0, ql, B, Lq, num_pages, page_size, max_blocks, Hq, Hkv, D, c, w, float(base),
        float(sm_scale or 0.0), code, ws.data_ptr(), nbytes, _stream(q.device)))
    return (o, lse) if return_lse else o


def selfextend_decode_workspace_bytes(kv_len, Hq, Hkv, D, group, window, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    kl, _ = _host_i64(kv_len, len(kv_len), "kv_len")
    return int(_lib.load().dca_selfextend_decode_workspace_bytes(kl, len(kv_len), Hq, Hkv, D, group, window, code))


def coarse_fine_decode_workspace_bytes(kv_len, Hq, Hkv, D, chunk, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    kl, _ = _host_i64(kv_len, len(kv_len), "kv_len")
    return int(_lib.load().dca_coarse_fine_decode_workspace_bytes(kl, len(kv_len), Hq, Hkv, D, chunk, code))


def _map_decode(fn_ws, fn, q, k_cache, k2, v_cache, kv_len, params, base, sm_scale, return_lse, workspace, name):
    lib = _lib.load()
    _check(q, "q", 3)
    for t, n in ((k_cache, "k_cache"), (k2, name), (v_cache, "v_cache")):
        _check(t, n, 4, q.dtype)
    B, Hq, D = q.shape
    cache_len, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, cache_len, Hkv, D) or v_cache.shape != k_cache.shape or k2.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    code = _dtype_code(q)
    kl, _ = _host_i64(kv_len, B, "kv_len")
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = int(getattr(lib, fn_ws)(kl, B, Hq, Hkv, D, *params[0], code))
    if nbytes == 0:
        raise ValueError("invalid decode sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check(fn, getattr(lib, fn)(
        q.data_ptr(), k_cache.data_ptr(), k2.data_ptr(), v_cache.data_ptr(), o.data_ptr(), _ptr(lse), kl, B,
        cache_len, Hq, Hkv, D, *params[1], float(base), float(sm_scale or 0.0), code, ws.data_ptr(), nbytes,
        _stream(q.device)))
    return (o, lse) if return_lse else o


def selfextend_decode(q, k_cache, k_cache_grouped, v_cache, kv_len, group: int, window: int,
                      base: float = 10000.0, sm_scale: float | None = None, return_lse: bool = False,
                      workspace=None):
    """SelfExtend decode of a ragged batch: q [B, Hq, D] raw; k_cache rotated at j,
    k_cache_grouped at floor(j / group), v_cache: [B, cache_len, Hkv, D]."""
    return _map_decode("dca_selfextend_decode_workspace_bytes", "dca_selfextend_decode", q, k_cache,
                       k_cache_grouped, v_cache, kv_len, ((group, window), (group, window)), base, sm_scale,
                       return_lse, workspace, "k_cache_grouped")


def coarse_fine_decode(q, k_cache, k_cache_scaled, v_cache, kv_len, chunk: int, train_len: int, target_len: int,
                       base: float = 10000.0, sm_scale: float | None = None, return_lse: bool = False,
                       workspace=None):
    """Coarse / fine map decode of a ragged batch: k_cache rotated at j, k_cache_scaled
    at floor(j / chunk) * chunk * train_len / target_len + j mod chunk."""
    return _map_decode("dca_coarse_fine_decode_workspace_bytes", "dca_coarse_fine_decode", q, k_cache,
                       k_cache_scaled, v_cache, kv_len, ((chunk,), (chunk, train_len, target_len)), base,
                       sm_scale, return_lse, workspace, "k_cache_scaled")


def _map_decode_paged(fn_ws, fn, q, k_pages, k2_pages, v_pages, block_table, kv_len, params, base, sm_scale,
                      return_lse, workspace, name):
    lib = _lib.load()
    _check(q, "q", 3)
    num_pages, page_size, Hkv, max_blocks = _check_pages(k_pages, v_pages, block_table, q)
    _check(k2_pages, name, 4, q.dtype)
    if k2_pages.shape != k_pages.shape:
        raise ValueError(f"{name} and k_pages differ in shape")
    B, Hq, D = q.shape
    if k_pages.shape[3] != D or block_table.shape[0] != B:
        raise ValueError("page pool / block table shapes do not match q")
    code = _dtype_code(q)
    kl, _ = _host_i64(kv_len, B, "kv_len")
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = int(getattr(lib, fn_ws)(kl, B, Hq, Hkv, D, *params[0], code))
    if nbytes == 0:
        raise ValueError("invalid decode sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check(fn, getattr(lib, fn)(
        q.data_ptr(), k_pages.data_ptr(), k2_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
        o.data_ptr(), _ptr(lse), kl, B, num_pages, page_size, max_blocks, Hq, Hkv, D, *params[1], float(base),
        float(sm_scale or 0.0), code, ws.data_ptr(), nbytes, _stream(q.device)))
    return (o, lse) if return_lse else o


def selfextend_decode_paged(q, k_pages, k_pages_grouped, v_pages, block_table, kv_len, group: int, window: int,
                            base: float = 10000.0, sm_scale: float | None = None, return_lse: bool = False,
                            workspace=None):
    """selfextend_decode over page pools [num_pages, page_size, Hkv, D] (keys at j, keys
    at floor(j / group), values) sharing one int32 block table [B, max_blocks]."""
    return _map_decode_paged("dca_selfextend_decode_workspace_bytes", "dca_selfextend_decode_paged", q, k_pages,
                             k_pages_grouped, v_pages, block_table, kv_len, ((group, window), (group, window)),
                             base, sm_scale, return_lse, workspace, "k_pages_grouped")


def coarse_fine_decode_paged(q, k_pages, k_pages_scaled, v_pages, block_table, kv_len, chunk: int, train_len: int,
                             target_len: int, base: float = 10000.0, sm_scale: float | None = None,
                             return_lse: bool = False, workspace=None):
    """coarse_fine_decode over page pools (keys at j, coarse-scaled keys, values) sharing
    one int32 block table [B, max_blocks]."""
    return _map_decode_paged("dca_coarse_fine_decode_workspace_bytes", "dca_coarse_fine_decode_paged", q, k_pages,
                             k_pages_scaled, v_pages, block_table, kv_len, ((chunk,), (chunk, train_len, target_len)),
                             base, sm_scale, return_lse, workspace, "k_pages_scaled")


def coarse_fine_key_remap(x, chunk: int, train_len: int, target_len: int, base: float = 10000.0, pos0: int = 0,
                          out=None):
    """Rotate x [B, L, H, D] (positions pos0 ..) at the coarse-scaled key positions."""
    lib = _lib.load()
    _check(x, "x", 4)
    B, L, H, D = x.shape
    out = torch.empty_like(x) if out is None else out
    _check_out(out, "out", x.shape, x.dtype, x.device)
    _lib.check("dca_coarse_fine_key_remap", lib.dca_coarse_fine_key_remap(
        x.data_ptr(), out.data_ptr(), B, L, H, D, int(pos0), chunk, train_len, target_len, float(base),
        _dtype_code(x), _stream(x.device)))
    return out


def coarse_fine_prefill(q, k, v, chunk: int, train_len: int, target_len: int, base: float = 10000.0,
                        sm_scale: float | None = None, return_lse: bool = False, workspace=None):
    """Causal prefill under the DCA guide's coarse / fine distance map (chunk size,
    coarse distance scaled by train_len / target_len, lambda ramp for adjacent chunks).
    q [B, L, Hq, D], k/v [B, L, Hkv, D] raw; returns o (and lse)."""
    lib = _lib.load()
    _check(q, "q", 4)
    _check(k, "k", 4, q.dtype)
    _check(v, "v", 4, q.dtype)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, L, Hkv, D) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    code = _dtype_code(q)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, L, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = int(lib.dca_coarse_fine_workspace_bytes(B, L, Hkv, D, code))
    if nbytes == 0:
        raise ValueError("invalid coarse / fine prefill sizes")
    ws = _workspace(nbytes, q.device, workspace)
    _lib.check("dca_coarse_fine_prefill", lib.dca_coarse_fine_prefill(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse), B, L, Hq, Hkv, D,
        chunk, train_len, target_len, float(base), float(sm_scale or 0.0), code,
        ws.data_ptr(), nbytes, _stream(q.device)))
    return (o, lse) if return_lse else o


# ---- the C entry points under their own names (include/dca.h) ----------------------
# The same marshalling functions as above: tensors in, the C call on torch's
# current stream, tensors out.
def dca_status_string(status: int) -> str:
    return _lib.load().dca_status_string(int(status)).decode()


def dca_version() -> int:
    return int(_lib.load().dca_version())


dca_rope_remap = rope_remap
dca_prefill = prefill
dca_prefill_prepare = prefill_prepare
dca_prefill_attend = prefill_attend
dca_prefill_workspace_bytes = prefill_workspace_bytes
dca_decode = decode
dca_decode_workspace_bytes = decode_workspace_bytes
dca_selfextend_prefill = selfextend_prefill
dca_selfextend_workspace_bytes = selfextend_workspace_bytes
dca_prefill_chunk = prefill_chunk
dca_decode_varlen = decode_varlen
dca_decode_varlen_workspace_bytes = decode_varlen_workspace_bytes
dca_decode_paged = decode_paged
dca_decode_paged_noalloc = decode_paged_noalloc
dca_prefill_chunk_paged = prefill_chunk_paged
dca_coarse_fine_prefill = coarse_fine_prefill
dca_coarse_fine_workspace_bytes = coarse_fine_workspace_bytes
dca_selfextend_decode = selfextend_decode
dca_selfextend_decode_workspace_bytes = selfextend_decode_workspace_bytes
dca_coarse_fine_decode = coarse_fine_decode
dca_coarse_fine_decode_workspace_bytes = coarse_fine_decode_workspace_bytes
dca_selfextend_decode_paged = selfextend_decode_paged
dca_coarse_fine_decode_paged = coarse_fine_decode_paged
dca_coarse_fine_key_remap = coarse_fine_key_remap

__all__ += [n for n in list(globals()) if n.startswith("dca_")]
