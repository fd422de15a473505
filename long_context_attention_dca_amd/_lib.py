"""ctypes view of the C ABI in include/dca.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libdca_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

DCA_F32 = 0
DCA_BF16 = 1
DCA_MAP_KEY = 0
DCA_MAP_Q_INTRA = 1
DCA_MAP_Q_SUCC = 2
DCA_MAP_Q_INTER = 3
DCA_MAP_PLAIN = 4
DCA_MAP_SE_KEY_GROUPED = 5
DCA_MAP_SE_Q_GROUPED = 6
DCA_OK = 0
DCA_ERR_INVALID_ARG = -1
DCA_ERR_UNSUPPORTED = -2
DCA_ERR_WORKSPACE = -3
DCA_ERR_HIP = -4
DCA_ERR_TOO_LARGE = -5
DCA_NOALLOC_SCRATCH_BYTES = 32 << 20

_i64, _int, _dbl, _flt, _vp, _sz = (ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_float,
                                    ctypes.c_void_p, ctypes.c_size_t)
_fp = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)   # host int64 arrays

# name -> (restype, argtypes); the exported surface of include/dca.h
SIGNATURES = {
    "dca_status_string": (ctypes.c_char_p, [_int]),
    "dca_version": (_int, []),
    "dca_rope_remap": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _int, _dbl, _int, _vp]),
    "dca_prefill_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _int, _int]),
    "dca_prefill": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int,
                           _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_prefill_prepare": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _dbl, _int, _vp,
                                   _sz, _vp]),
    "dca_prefill_attend": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _flt, _int,
                                  _vp, _sz, _vp]),
    "dca_selfextend_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _int, _int, _int]),
    "dca_selfextend_prefill": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int,
                                      _int, _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_coarse_fine_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _int]),
    "dca_coarse_fine_prefill": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int,
                                       _int, _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_prefill_chunk": (_int, [_vp, _vp, _vp, _vp, _vp, _i64p, _i64p, _i64, _i64, _i64, _i64, _i64,
                                 _i64, _int, _int, _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_decode_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _int]),
    "dca_decode_varlen_workspace_bytes": (_sz, [_i64p, _i64, _i64, _i64, _i64, _int]),
    "dca_decode_varlen": (_int, [_vp, _vp, _vp, _vp, _vp, _i64p, _i64, _i64, _i64, _i64, _i64, _int, _int,
                                 _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_decode": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _dbl,
                          _flt, _int, _vp, _sz, _vp]),
    "dca_decode_paged": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64, _i64, _i64, _i64, _i64, _i64,
                                _i64, _int, _int, _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_decode_paged_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64, _i64, _i64, _i64, _i64, _i64,
                                        _i64, _int, _int, _dbl, _flt, _int, _vp]),
    "dca_prefill_chunk_paged": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64p, _i64, _i64, _i64, _i64,
                                       _i64, _i64, _i64, _i64, _int, _int, _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_selfextend_decode_workspace_bytes": (_sz, [_i64p, _i64, _i64, _i64, _i64, _int, _int, _int]),
    "dca_selfextend_decode": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64, _i64, _i64, _i64, _i64, _int,
                                     _int, _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_coarse_fine_decode_workspace_bytes": (_sz, [_i64p, _i64, _i64, _i64, _i64, _int, _int]),
    "dca_coarse_fine_decode": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64, _i64, _i64, _i64, _i64, _int,
                                      _int, _int, _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_coarse_fine_key_remap": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _int, _dbl, _int,
                                         _vp]),
    "dca_selfextend_decode_paged": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64, _i64, _i64, _i64, _i64,
                                           _i64, _i64, _int, _int, _dbl, _flt, _int, _vp, _sz, _vp]),
    "dca_coarse_fine_decode_paged": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64, _i64, _i64, _i64, _i64,
                                            _i64, _i64, _int, _int, _int, _dbl, _flt, _int, _vp, _sz, _vp]),
}

_lib = None


class DCAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build the HIP library first "
            "(python -m long_context_attention_dca_amd.build); there is no fallback path")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().dca_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != DCA_OK:
        raise DCAError(fn, status)
