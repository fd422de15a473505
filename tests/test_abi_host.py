"""Host-only checks of the C ABI: the library loads without a GPU, exports every
symbol include/dca.h declares, and rejects invalid calls before any HIP call.

No call here passes validation, so nothing touches a device (the fake
pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

from long_context_attention_dca_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dca.h")
FAKE = 0x10000  # 16-byte aligned, never dereferenced
FAKE_WS = 0x100000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from long_context_attention_dca_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dca_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_python_binding_has_every_entry_point_by_name(lib):
    # the binding exposes each C entry point under its own name (tensors in,
    # the C call, tensors out)
    import long_context_attention_dca_amd as dca
    for name in declared_functions():
        assert callable(getattr(dca, name, None)), name
    assert dca.dca_version() == 10000
    assert dca.dca_status_string(-3).startswith("DCA_ERR_WORKSPACE")


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings_and_version(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.dca_status_string(code).decode().startswith("DCA_")
    assert lib.dca_status_string(12345).decode() == "unknown DCA status"
    assert lib.dca_version() == 10000


def test_prefill_workspace_sizes(lib):
    # fp32, B=1, L=512, Hkv=1, D=64, c=128: fp64 table 128*32*16 B, rotated keys 512*64*4 B.
    assert lib.dca_prefill_workspace_bytes(1, 512, 1, 64, 128, 0) == 128 * 32 * 16 + 2 * 512 * 64 * 4
    # plus the values (bf16: tiled transpose); L is padded to a multiple of 128 rows.
    n = lib.dca_prefill_workspace_bytes(2, 100, 3, 128, 4096, 1)
    assert n == 4096 * 64 * 16 + 2 * (2 * 3 * 128 * 128 * 2)
    for bad in [(0, 512, 1, 64, 128, 0), (1, 0, 1, 64, 128, 0), (1, 512, 1, 96, 128, 0),
                (1, 512, 1, 64, 128, 7), (1, 512, 0, 64, 128, 1)]:
        assert lib.dca_prefill_workspace_bytes(*bad) == 0


def test_prefill_family_size_limits(lib):
    # B and Hkv index grid dimensions (at most 65535); beyond, every size query
    # of the prefill family returns 0 instead of a size the launch cannot use
    assert lib.dca_prefill_workspace_bytes(65535, 1, 1, 64, 128, 1) > 0
    assert lib.dca_prefill_workspace_bytes(65536, 1, 1, 64, 128, 1) == 0
    assert lib.dca_prefill_workspace_bytes(1, 1, 65536, 64, 128, 1) == 0
    assert lib.dca_selfextend_workspace_bytes(65536, 10, 1, 64, 4, 8, 1) == 0
    assert lib.dca_selfextend_workspace_bytes(65535, 10, 1, 64, 4, 8, 1) > 0
    assert lib.dca_coarse_fine_workspace_bytes(1, 10, 65536, 64, 1) == 0
    assert lib.dca_coarse_fine_workspace_bytes(1, 10, 65535, 64, 1) > 0
    # a padded key copy past 2^56 bytes is refused rather than wrapped
    assert lib.dca_prefill_workspace_bytes(65535, (1 << 30) - 1, 65535, 128, 128, 1) == 0


@pytest.mark.parametrize("D,dtype,limit", [(128, 1, 1 << 23), (64, 1, 1 << 24), (128, 0, 1 << 22),
                                           (64, 0, 1 << 23)])
def test_prefill_head_bytes_limit(lib, D, dtype, limit):
    # One head's padded key rows (a multiple of 128 rows) must stay below 2^31
    # bytes, so the attention kernel's 32-bit buffer offsets cannot wrap.
    # The size queries return 0 from there on, and the calls refuse it before
    # any HIP call; the largest accepted length is limit - 128.
    ok, bad = limit - 128, limit - 127          # bad pads up to `limit` rows
    for L in (ok,):
        assert lib.dca_prefill_workspace_bytes(1, L, 1, D, 4096, dtype) > 0
        assert lib.dca_selfextend_workspace_bytes(1, L, 1, D, 8, 1024, dtype) > 0
        assert lib.dca_coarse_fine_workspace_bytes(1, L, 1, D, dtype) > 0
    for L in (bad, limit, limit + 1000):
        assert lib.dca_prefill_workspace_bytes(1, L, 1, D, 4096, dtype) == 0
        assert lib.dca_selfextend_workspace_bytes(1, L, 1, D, 8, 1024, dtype) == 0
        assert lib.dca_coarse_fine_workspace_bytes(1, L, 1, D, dtype) == 0
        assert call_prefill(lib, L=L, D=D, dtype=dtype, Hq=1, Hkv=1, c=4096, w=1024,
                            ws_bytes=1 << 62) == _lib.DCA_ERR_INVALID_ARG
    # the chunked prefill counts the largest pos0 + q_len as the length
    assert call_chunk(lib, pos0=(0, limit - 64), Lq=64, cache_len=limit, D=D, dtype=dtype,
                      ws_bytes=1 << 62) == _lib.DCA_ERR_INVALID_ARG


def test_decode_workspace_sizes(lib):
    n = lib.dca_decode_workspace_bytes(16, 100001, 64, 8, 128, 1)
    assert n > 16 * 64 * 3 * 128 * 2
    assert n % 256 == 0
    assert lib.dca_decode_workspace_bytes(1, 10, 6, 4, 128, 1) == 0   # Hq % Hkv
    assert lib.dca_decode_workspace_bytes(1, 0, 8, 8, 128, 1) == 0


PREFILL_OK = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, k_rot_out=None, B=1, L=256, Hq=4, Hkv=2,
                  D=128, c=128, w=32, base=10000.0, sm_scale=0.0, dtype=1, ws=FAKE_WS, ws_bytes=1 << 30,
                  stream=None)


def call_prefill(lib, **over):
    a = dict(PREFILL_OK, **over)
    return lib.dca_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["k_rot_out"], a["B"], a["L"],
                           a["Hq"], a["Hkv"], a["D"], a["c"], a["w"], a["base"], a["sm_scale"],
                           a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), _lib.DCA_ERR_INVALID_ARG),
    (dict(v=None), _lib.DCA_ERR_INVALID_ARG),
    (dict(o=None), _lib.DCA_ERR_INVALID_ARG),
    (dict(D=96), _lib.DCA_ERR_UNSUPPORTED),
    (dict(dtype=2), _lib.DCA_ERR_UNSUPPORTED),
    (dict(w=128), _lib.DCA_ERR_INVALID_ARG),
    (dict(w=-1), _lib.DCA_ERR_INVALID_ARG),
    (dict(c=0, w=0), _lib.DCA_ERR_INVALID_ARG),
    (dict(Hq=3), _lib.DCA_ERR_INVALID_ARG),
    (dict(L=0), _lib.DCA_ERR_INVALID_ARG),
    (dict(B=0), _lib.DCA_ERR_INVALID_ARG),
    (dict(base=0.0), _lib.DCA_ERR_INVALID_ARG),
    (dict(base=float("nan")), _lib.DCA_ERR_INVALID_ARG),
    (dict(sm_scale=float("inf")), _lib.DCA_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), _lib.DCA_ERR_INVALID_ARG),
    (dict(k_rot_out=FAKE + 4), _lib.DCA_ERR_INVALID_ARG),
    (dict(ws=None), _lib.DCA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), _lib.DCA_ERR_WORKSPACE),
    (dict(ws=FAKE_WS + 16), _lib.DCA_ERR_WORKSPACE),
])
def test_prefill_rejects_before_touching_device(lib, over, status):
    assert call_prefill(lib, **over) == status


DECODE_OK = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=2, kv_len=1000, Hq=8, Hkv=2, D=64, c=128,
                 w=32, base=10000.0, sm_scale=0.0, dtype=1, ws=FAKE_WS, ws_bytes=1 << 30, stream=None)


def call_decode(lib, **over):
    a = dict(DECODE_OK, **over)
    return lib.dca_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["kv_len"], a["Hq"],
                          a["Hkv"], a["D"], a["c"], a["w"], a["base"], a["sm_scale"], a["dtype"], a["ws"],
                          a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(k=None), _lib.DCA_ERR_INVALID_ARG),
    (dict(D=32), _lib.DCA_ERR_UNSUPPORTED),
    (dict(w=200), _lib.DCA_ERR_INVALID_ARG),
    (dict(Hkv=3), _lib.DCA_ERR_INVALID_ARG),
    (dict(kv_len=0), _lib.DCA_ERR_INVALID_ARG),
    (dict(lse=FAKE + 2), _lib.DCA_ERR_INVALID_ARG),
    (dict(ws_bytes=0), _lib.DCA_ERR_WORKSPACE),
])
def test_decode_rejects_before_touching_device(lib, over, status):
    assert call_decode(lib, **over) == status


@pytest.mark.parametrize("args,status", [
    ((None, FAKE, 1, 8, 2, 64, 0, 0, 128, 32, 1e4, 1, None), _lib.DCA_ERR_INVALID_ARG),
    ((FAKE, FAKE, 1, 8, 2, 80, 0, 0, 128, 32, 1e4, 1, None), _lib.DCA_ERR_UNSUPPORTED),
    ((FAKE, FAKE, 1, 8, 2, 64, 0, 9, 128, 32, 1e4, 1, None), _lib.DCA_ERR_INVALID_ARG),
    ((FAKE, FAKE, 1, 8, 2, 64, -1, 0, 128, 32, 1e4, 1, None), _lib.DCA_ERR_INVALID_ARG),
    ((FAKE, FAKE, 1, 8, 2, 64, 0, 0, 128, 128, 1e4, 1, None), _lib.DCA_ERR_INVALID_ARG),
    ((FAKE, FAKE + 2, 1, 8, 2, 64, 0, 0, 128, 32, 1e4, 1, None), _lib.DCA_ERR_INVALID_ARG),
    ((FAKE, FAKE, 0, 8, 2, 64, 0, 0, 128, 32, 1e4, 1, None), _lib.DCA_OK),   # empty: no-op
    ((FAKE, FAKE, 1, 8, 1 << 25, 64, 0, 0, 128, 32, 1e4, 1, None), _lib.DCA_ERR_INVALID_ARG),  # H * D = 2^31
])
def test_remap_validation(lib, args, status):
    assert lib.dca_rope_remap(*args) == status


def test_two_phase_prefill_validation(lib):
    # prepare: k, v, k_rot_out, B, L, Hkv, D, c, w, base, dtype, ws, ws_bytes, stream
    ok = [FAKE, FAKE, None, 1, 256, 2, 128, 128, 32, 1e4, 1, FAKE_WS, 1 << 30, None]
    for i, bad, st in [(0, None, -1), (4, 0, -1), (6, 80, -2), (8, 128, -1), (9, -1.0, -1),
                       (11, None, -3), (12, 16, -3)]:
        a = list(ok)
        a[i] = bad
        assert lib.dca_prefill_prepare(*a) == st, (i, bad)
    # attend: q, o, lse, B, L, Hq, Hkv, D, c, w, sm_scale, dtype, ws, ws_bytes, stream
    ok = [FAKE, FAKE, None, 1, 256, 4, 2, 128, 128, 32, 0.0, 1, FAKE_WS, 1 << 30, None]
    for i, bad, st in [(0, None, -1), (1, FAKE + 4, -1), (5, 3, -1), (7, 48, -2), (9, 200, -1),
                       (10, float("nan"), -1), (12, None, -3)]:
        a = list(ok)
        a[i] = bad
        assert lib.dca_prefill_attend(*a) == st, (i, bad)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "missing.so"))


def test_selfextend_workspace_sizes(lib):
    # bf16, B 2, L 100, Hkv 3, D 128, G 4, W 16: positions up to max(99, 99//4 + 16 - 4) = 99
    Lp = 128
    table = 100 * 64 * 16
    kbytes = 2 * 3 * Lp * 128 * 2
    want = table + 3 * kbytes          # (each piece is already a multiple of 256)
    assert lib.dca_selfextend_workspace_bytes(2, 100, 3, 128, 4, 16, 1) == want
    # a wide window pushes the grouped query position past L - 1: 99//4 + 300 - 75 = 249
    assert lib.dca_selfextend_workspace_bytes(2, 100, 3, 128, 4, 300, 1) == 250 * 64 * 16 + 3 * kbytes
    assert lib.dca_selfextend_workspace_bytes(1, 100, 1, 128, 0, 16, 1) == 0    # group < 1
    assert lib.dca_selfextend_workspace_bytes(1, 100, 1, 128, 4, -1, 1) == 0    # window < 0
    assert lib.dca_selfextend_workspace_bytes(1, 100, 1, 96, 4, 16, 1) == 0     # head dim


SE_OK = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, L=256, Hq=4, Hkv=2, D=128, G=4, W=32,
             base=10000.0, sm_scale=0.0, dtype=1, ws=FAKE_WS, ws_bytes=1 << 30, stream=None)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), _lib.DCA_ERR_INVALID_ARG),
    (dict(k=None), _lib.DCA_ERR_INVALID_ARG),
    (dict(G=0), _lib.DCA_ERR_INVALID_ARG),
    (dict(W=-3), _lib.DCA_ERR_INVALID_ARG),
    (dict(Hq=3), _lib.DCA_ERR_INVALID_ARG),
    (dict(L=0), _lib.DCA_ERR_INVALID_ARG),
    (dict(D=80), _lib.DCA_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.DCA_ERR_UNSUPPORTED),
    (dict(lse=FAKE + 1), _lib.DCA_ERR_INVALID_ARG),
    (dict(base=-1.0), _lib.DCA_ERR_INVALID_ARG),
    (dict(ws_bytes=4096), _lib.DCA_ERR_WORKSPACE),
    (dict(ws=None), _lib.DCA_ERR_WORKSPACE),
])
def test_selfextend_rejects_before_touching_device(lib, over, status):
    a = dict(SE_OK, **over)
    assert lib.dca_selfextend_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["L"], a["Hq"],
                                      a["Hkv"], a["D"], a["G"], a["W"], a["base"], a["sm_scale"],
                                      a["dtype"], a["ws"], a["ws_bytes"], a["stream"]) == status


@pytest.mark.parametrize("map_,c,w,status", [
    (_lib.DCA_MAP_SE_KEY_GROUPED, 4, 100, _lib.DCA_OK),      # w >= c is fine for the grouped maps
    (_lib.DCA_MAP_SE_Q_GROUPED, 1, 0, _lib.DCA_OK),
    (_lib.DCA_MAP_SE_KEY_GROUPED, 0, 8, _lib.DCA_ERR_INVALID_ARG),
    (_lib.DCA_MAP_SE_Q_GROUPED, 4, -1, _lib.DCA_ERR_INVALID_ARG),
    (7, 4, 8, _lib.DCA_ERR_INVALID_ARG),
    (_lib.DCA_MAP_KEY, 4, 8, _lib.DCA_ERR_INVALID_ARG),         # DCA maps still need w < c
])
def test_remap_selfextend_map_validation(lib, map_, c, w, status):
    # B = 0: a valid call is an empty no-op, so nothing reaches the device
    assert lib.dca_rope_remap(FAKE, FAKE, 0, 8, 2, 64, 0, map_, c, w, 1e4, 1, None) == status


def _i64s(*vals):
    import ctypes
    return (ctypes.c_int64 * len(vals))(*vals)


CHUNK_OK = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, pos0=(0, 64), q_len=None, B=2, Lq=64,
                cache_len=256, Hq=4, Hkv=2, D=128, c=128, w=32, base=1e4, sm_scale=0.0, dtype=1,
                ws=FAKE_WS, ws_bytes=1 << 30, stream=None)


def call_chunk(lib, **over):
    a = dict(CHUNK_OK, **over)
    p0 = None if a["pos0"] is None else _i64s(*a["pos0"])
    ql = None if a["q_len"] is None else _i64s(*a["q_len"])
    return lib.dca_prefill_chunk(a["q"], a["k"], a["v"], a["o"], a["lse"], p0, ql, a["B"], a["Lq"],
                                 a["cache_len"], a["Hq"], a["Hkv"], a["D"], a["c"], a["w"], a["base"],
                                 a["sm_scale"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(pos0=None), _lib.DCA_ERR_INVALID_ARG),
    (dict(pos0=(0, -1)), _lib.DCA_ERR_INVALID_ARG),
    (dict(pos0=(0, 200)), _lib.DCA_ERR_INVALID_ARG),        # 200 + 64 > cache_len
    (dict(q_len=(65, 1)), _lib.DCA_ERR_INVALID_ARG),        # more rows than Lq
    (dict(q_len=(-1, 1)), _lib.DCA_ERR_INVALID_ARG),
    (dict(Lq=300), _lib.DCA_ERR_INVALID_ARG),               # Lq > cache_len
    (dict(k=None), _lib.DCA_ERR_INVALID_ARG),
    (dict(w=128), _lib.DCA_ERR_INVALID_ARG),
    (dict(D=96), _lib.DCA_ERR_UNSUPPORTED),
    (dict(ws_bytes=100), _lib.DCA_ERR_WORKSPACE),
    (dict(q_len=(0, 0)), _lib.DCA_OK),                      # no rows: nothing enqueued
])
def test_prefill_chunk_validation(lib, over, status):
    assert call_chunk(lib, **over) == status


@pytest.mark.parametrize("kv,status", [((0, 5), _lib.DCA_ERR_INVALID_ARG), ((5, 1001), _lib.DCA_ERR_INVALID_ARG),
                                       (None, _lib.DCA_ERR_INVALID_ARG)])
def test_decode_varlen_validation(lib, kv, status):
    arr = None if kv is None else _i64s(*kv)
    assert lib.dca_decode_varlen(FAKE, FAKE, FAKE, FAKE, None, arr, 2, 1000, 8, 2, 64, 128, 32, 1e4, 0.0, 1,
                                 FAKE_WS, 1 << 30, None) == status
    assert lib.dca_decode_varlen(FAKE, FAKE, FAKE, FAKE, None, _i64s(5, 9), 2, 1000, 8, 2, 64, 128, 32, 1e4,
                                 0.0, 1, FAKE_WS, 64, None) == _lib.DCA_ERR_WORKSPACE


def test_decode_varlen_workspace_sizes(lib):
    # uniform lengths give the uniform layout
    assert lib.dca_decode_varlen_workspace_bytes(_i64s(*([100001] * 16)), 16, 64, 8, 128, 1) == \
        lib.dca_decode_workspace_bytes(16, 100001, 64, 8, 128, 1)
    # a ragged batch spreads its keys: at least as many ranges for the longest sequence
    ragged = lib.dca_decode_varlen_workspace_bytes(_i64s(*([1000] * 15 + [100001])), 16, 64, 8, 128, 1)
    assert ragged >= lib.dca_decode_workspace_bytes(16, 100001, 64, 8, 128, 1)
    assert lib.dca_decode_varlen_workspace_bytes(_i64s(5, 0), 2, 8, 2, 64, 1) == 0
    assert lib.dca_decode_varlen_workspace_bytes(None, 2, 8, 2, 64, 1) == 0


def test_coarse_fine_workspace_and_validation(lib):
    Lp = 128
    kbytes = 2 * 3 * Lp * 128 * 2
    # theta table, then the (cos, sin) of the 3 query positions of 100 rows, then keys twice and V
    assert lib.dca_coarse_fine_workspace_bytes(2, 100, 3, 128, 1) == 512 + 3 * 100 * 64 * 16 + 3 * kbytes
    assert lib.dca_coarse_fine_workspace_bytes(2, 100, 3, 96, 1) == 0
    ok = [FAKE, FAKE, FAKE, FAKE, None, 1, 256, 4, 2, 128, 512, 4096, 32768, 1e4, 0.0, 1, FAKE_WS, 1 << 30, None]
    for i, bad, st in [(0, None, -1), (10, 0, -1), (11, 0, -1), (12, -5, -1), (10, 96, -2), (9, 80, -2),
                       (17, 64, -3), (13, 0.0, -1)]:
        a = list(ok)
        a[i] = bad
        assert lib.dca_coarse_fine_prefill(*a) == st, (i, bad)


def test_decode_paged_validation(lib):
    # q, k_pages, v_pages, block_table, o, lse, kv_len, B, num_pages, page_size, max_blocks, Hq, Hkv, D,
    # c, w, base, sm_scale, dtype, ws, ws_bytes, stream
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, None, _i64s(40, 100), 2, 20, 16, 8, 8, 2, 64, 128, 32, 1e4, 0.0, 1,
          FAKE_WS, 1 << 30, None]
    for i, bad, st in [(3, None, -1),            # no block table
                       (9, 8, -1), (9, 24, -1), (9, 0, -1),   # page size not a multiple of 16
                       (8, 0, -1), (10, 0, -1),  # empty pool / table
                       (6, _i64s(40, 129), -1),  # 129 rows > 8 blocks of 16
                       (6, _i64s(0, 5), -1),
                       (13, 96, -2), (18, 3, -2),
                       (20, 64, -3), (19, None, -3)]:
        a = list(ok)
        a[i] = bad
        assert lib.dca_decode_paged(*a) == st, (i, bad)


def test_decode_paged_noalloc_validation(lib):
    # Same arguments as dca_decode_paged without (ws, ws_bytes).  Invalid calls,
    # and calls that need more than the static scratch, return before any HIP
    # call (the fake pointers are never touched).
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, None, _i64s(40, 100), 2, 20, 16, 8, 8, 2, 64, 128, 32, 1e4, 0.0, 1, None]
    for i, bad, st in [(3, None, -1), (0, None, -1), (4, None, -1), (9, 8, -1), (8, 0, -1),
                       (6, _i64s(40, 129), -1), (6, None, -1), (13, 96, -2), (18, 3, -2), (15, 128, -1),
                       (0, FAKE + 8, -1)]:
        a = list(ok)
        a[i] = bad
        assert lib.dca_decode_paged_noalloc(*a) == st, (i, bad)
    # 64 sequences x 1024 query heads: the rotated query variants alone take
    # 64 * 1024 * 3 * 128 * 2 bytes > 32 MiB
    big = [FAKE, FAKE, FAKE, FAKE, FAKE, None, _i64s(*([1000] * 64)), 64, 4096, 16, 64, 1024, 8, 128, 4096,
           1024, 1e4, 0.0, 1, None]
    need = lib.dca_decode_varlen_workspace_bytes(_i64s(*([1000] * 64)), 64, 1024, 8, 128, 1)
    assert need > _lib.DCA_NOALLOC_SCRATCH_BYTES
    assert lib.dca_decode_paged_noalloc(*big) == _lib.DCA_ERR_TOO_LARGE
    assert lib.dca_status_string(_lib.DCA_ERR_TOO_LARGE).decode().startswith("DCA_ERR_TOO_LARGE")


def test_noalloc_scratch_constant_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define DCA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.DCA_NOALLOC_SCRATCH_BYTES
    assert "#define DCA_ERR_TOO_LARGE (-5)" in text and _lib.DCA_ERR_TOO_LARGE == -5


def test_prefill_chunk_paged_validation(lib):
    # q, k_pages, v_pages, block_table, o, lse, pos0, q_len, B, Lq, num_pages, page_size, max_blocks,
    # Hq, Hkv, D, c, w, base, sm_scale, dtype, ws, ws_bytes, stream
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, None, _i64s(32, 64), None, 2, 32, 20, 32, 4, 8, 2, 128, 256, 64, 1e4,
          0.0, 1, FAKE_WS, 1 << 30, None]
    for i, bad, st in [(3, None, -1), (11, 17, -1), (12, 0, -1),
                       (6, _i64s(32, 97), -1),   # 97 + 32 rows > 4 blocks of 32
                       (6, _i64s(-1, 0), -1),
                       (15, 80, -2), (22, 64, -3)]:
        a = list(ok)
        a[i] = bad
        assert lib.dca_prefill_chunk_paged(*a) == st, (i, bad)
    # no rows at all: nothing to do, no device call
    a = list(ok)
    a[7] = _i64s(0, 0)
    assert lib.dca_prefill_chunk_paged(*a) == 0


def test_map_decode_workspace_and_validation(lib):
    kv = _i64s(100, 3000, 777)
    # a window covering every cache: one segment, the DCA ragged plan
    assert lib.dca_selfextend_decode_workspace_bytes(kv, 3, 16, 2, 128, 4, 10 ** 6, 1) == \
        lib.dca_decode_varlen_workspace_bytes(kv, 3, 16, 2, 128, 1)
    # two segments: at least as many partials
    assert lib.dca_selfextend_decode_workspace_bytes(kv, 3, 16, 2, 128, 4, 64, 1) >= \
        lib.dca_decode_varlen_workspace_bytes(kv, 3, 16, 2, 128, 1)
    assert lib.dca_coarse_fine_decode_workspace_bytes(kv, 3, 16, 2, 128, 64, 1) > 0
    assert lib.dca_selfextend_decode_workspace_bytes(kv, 3, 16, 2, 128, 0, 64, 1) == 0     # group 0
    assert lib.dca_coarse_fine_decode_workspace_bytes(kv, 3, 16, 2, 128, 0, 1) == 0        # chunk 0
    assert lib.dca_coarse_fine_decode_workspace_bytes(_i64s(5, 0), 2, 16, 2, 128, 64, 1) == 0
    # q, kc, kc2, vc, o, lse, kv_len, B, cache_len, Hq, Hkv, D, group, window, base, scale, dtype, ws, bytes, st
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, None, _i64s(40, 100), 2, 128, 8, 2, 64, 4, 16, 1e4, 0.0, 1,
          FAKE_WS, 1 << 30, None]
    for i, bad, st in [(2, None, -1), (12, 0, -1), (13, -1, -1), (6, _i64s(40, 129), -1), (11, 96, -2),
                       (16, 5, -2), (18, 64, -3)]:
        a = list(ok)
        a[i] = bad
        assert lib.dca_selfextend_decode(*a) == st, (i, bad)
    # ..., chunk, train_len, target_len, base, scale, dtype, ws, bytes, stream
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, None, _i64s(40, 100), 2, 128, 8, 2, 64, 64, 4, 32, 1e4, 0.0, 1,
          FAKE_WS, 1 << 30, None]
    for i, bad, st in [(2, None, -1), (12, 0, -1), (13, 0, -1), (14, 0, -1), (6, _i64s(0, 5), -1),
                       (11, 80, -2), (19, 64, -3)]:
        a = list(ok)
        a[i] = bad
        assert lib.dca_coarse_fine_decode(*a) == st, (i, bad)
    # x, out, B, L, H, D, pos0, chunk, train, target, base, dtype, stream
    ok = [FAKE, FAKE, 1, 10, 2, 64, 0, 16, 4, 32, 1e4, 1, None]
    for i, bad, st in [(0, None, -1), (7, 0, -1), (8, 0, -1), (6, -1, -1), (5, 48, -2), (10, -1.0, -1)]:
        a = list(ok)
        a[i] = bad
        assert lib.dca_coarse_fine_key_remap(*a) == st, (i, bad)
    a = list(ok)
    a[3] = 0   # no rows: nothing to do
    assert lib.dca_coarse_fine_key_remap(*a) == 0


@pytest.mark.parametrize("fn,params", [("dca_selfextend_decode_paged", (4, 100)),
                                       ("dca_coarse_fine_decode_paged", (64, 1, 8))])
def test_map_decode_paged_validation(lib, fn, params):
    # q, k_pages, k_pages_2nd, v_pages, block_table, o, lse, kv_len, B, num_pages, page_size, max_blocks,
    # Hq, Hkv, D, <map params>, base, sm_scale, dtype, ws, ws_bytes, stream
    n = len(params)
    ok = ([FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, _i64s(40, 100), 2, 20, 16, 8, 8, 2, 64] + list(params)
          + [1e4, 0.0, 1, FAKE_WS, 1 << 30, None])
    f = getattr(lib, fn)
    for i, bad, st in [(2, None, -1),            # no second key pool
                       (4, None, -1),            # no block table
                       (10, 24, -1),             # page size not a multiple of 16
                       (7, _i64s(40, 129), -1),  # 129 rows > 8 blocks of 16
                       (13, 3, -1),              # Hq % Hkv
                       (14, 96, -2), (17 + n, 3, -2),
                       (19 + n, 64, -3), (18 + n, None, -3)]:
        a = list(ok)
        a[i] = bad
        assert f(*a) == st, (fn, i, bad)
    a = list(ok)
    a[15] = 0            # SelfExtend group 0 / coarse-fine chunk 0
    assert f(*a) == -1
