"""Seeded random sweep of small shapes through every entry point, against the
fp64 oracle.

Each case draws its sizes from a fixed seed: lengths from 1 to several
hundred (tile multiples and ragged tails alike), GQA ratios 1 / 2 / 4, both
head dims, both dtypes, and the map parameters over their whole valid range
(chunk sizes that straddle tiles, w = 0, windows wider than the sequence,
group 1, chunk offsets that are and are not multiples of 32, page sizes
16 / 32 / 48 / 64), and the SelfExtend and coarse / fine decodes (dense, and
from page pools, which must give the same bits).  Inputs are the discriminating ones (q, k scaled by 2).
Bars: fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and mean-abs <= 2e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs
from test_gpu_parity import assert_close, dev, log, to_np
from test_gpu_paged import to_pages

pytestmark = pytest.mark.gpu

N_CASES = 24


def _draw(kind, idx):
    rng = np.random.default_rng(10_000 + 97 * idx + {"dca": 0, "se": 1, "cf": 2, "chunk": 3, "dec": 4,
                                                      "paged": 5, "sedec": 6, "cfdec": 7}[kind])
    dtype = torch.bfloat16 if idx % 4 != 3 else torch.float32
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 3))
    L = int(rng.choice([int(rng.integers(1, 80)), int(rng.integers(80, 400)), int(rng.integers(400, 700))]))
    return rng, dtype, D, Hkv, G, B, L


@pytest.mark.parametrize("idx", range(N_CASES))
def test_sweep_dca_prefill(idx):
    rng, dtype, D, Hkv, G, B, L = _draw("dca", idx)
    c = int(rng.integers(2, 600))
    w = int(rng.integers(0, c))
    log(f"[sweep dca] B{B} L{L} Hq{Hkv * G} Hkv{Hkv} D{D} c{c} w{w} {dtype}")
    q, k, v = inputs.prefill_inputs(B, L, Hkv * G, Hkv, D, dtype, seed=idx, qk_scale=2.0)
    o = dca.prefill(q.to(dev()), k.to(dev()), v.to(dev()), c, w)
    O, _ = oracle.dca_prefill_ref(q, k, v, c, w)
    assert_close(to_np(o), O, dtype, "dca")


@pytest.mark.parametrize("idx", range(N_CASES))
def test_sweep_selfextend_prefill(idx):
    rng, dtype, D, Hkv, G, B, L = _draw("se", idx)
    grp = int(rng.integers(1, 9))
    win = int(rng.choice([0, int(rng.integers(1, 300)), L + 5]))
    log(f"[sweep se] B{B} L{L} Hq{Hkv * G} Hkv{Hkv} D{D} G{grp} W{win} {dtype}")
    q, k, v = inputs.prefill_inputs(B, L, Hkv * G, Hkv, D, dtype, seed=100 + idx, qk_scale=2.0)
    o = dca.selfextend_prefill(q.to(dev()), k.to(dev()), v.to(dev()), grp, win)
    O, _ = oracle.selfextend_prefill_ref(q, k, v, grp, win)
    assert_close(to_np(o), O, dtype, "selfextend")


@pytest.mark.parametrize("idx", range(N_CASES))
def test_sweep_coarse_fine_prefill(idx):
    rng, dtype, D, Hkv, G, B, L = _draw("cf", idx)
    chunk = int(rng.choice([64, 128, 192, 256, 384])) if dtype == torch.bfloat16 else int(rng.integers(1, 200))
    train = int(rng.integers(1, 50))
    target = int(rng.integers(train, 8 * train + 1))
    log(f"[sweep cf] B{B} L{L} Hq{Hkv * G} Hkv{Hkv} D{D} C{chunk} {train}->{target} {dtype}")
    q, k, v = inputs.prefill_inputs(B, L, Hkv * G, Hkv, D, dtype, seed=200 + idx, qk_scale=2.0)
    o = dca.coarse_fine_prefill(q.to(dev()), k.to(dev()), v.to(dev()), chunk, train, target)
    O, _ = oracle.coarse_fine_prefill_ref(q, k, v, chunk, train, target)
    assert_close(to_np(o), O, dtype, "coarse_fine")


@pytest.mark.parametrize("idx", range(N_CASES))
def test_sweep_chunked_prefill(idx):
    rng, dtype, D, Hkv, G, B, L = _draw("chunk", idx)
    c = int(rng.choice([64, 128, 256, 96, 200]))
    w = int(rng.integers(0, c // 2 + 1))
    Lq = int(rng.integers(1, 200))
    aligned = idx % 2 == 0
    pos0 = [int(rng.integers(0, 300)) // (32 if aligned else 1) * (32 if aligned else 1) for _ in range(B)]
    ql = [int(rng.integers(0, Lq + 1)) for _ in range(B)]
    ql[0] = Lq
    cache_len = max(p + n for p, n in zip(pos0, ql))
    log(f"[sweep chunk] B{B} Lq{Lq} pos0 {pos0} q_len {ql} Hq{Hkv * G} Hkv{Hkv} D{D} c{c} w{w} {dtype}")
    qf, k, v = inputs.prefill_inputs(B, cache_len, Hkv * G, Hkv, D, dtype, seed=300 + idx, qk_scale=2.0)
    q = torch.zeros(B, Lq, Hkv * G, D, dtype=dtype)
    for b in range(B):
        q[b, : ql[b]] = qf[b, pos0[b]: pos0[b] + ql[b]]
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    o = to_np(dca.prefill_chunk(q.to(dev()), kc, v.to(dev()), pos0, c, w, q_len=ql))
    O, _ = oracle.dca_prefill_chunk_ref(q, k, v, pos0, c, w, q_len=ql)
    for b in range(B):
        if ql[b]:
            assert_close(o[b, : ql[b]], O[b, : ql[b]], dtype, f"chunk seq {b}")


@pytest.mark.parametrize("idx", range(N_CASES))
def test_sweep_decode(idx):
    rng, dtype, D, Hkv, G, B, L = _draw("dec", idx)
    B = int(rng.integers(1, 6))
    c = int(rng.integers(2, 3000))
    w = int(rng.integers(0, c))
    kv = [int(rng.integers(1, 2500)) for _ in range(B)]
    cache_len = max(kv)
    log(f"[sweep decode] kv {kv} Hq{Hkv * G} Hkv{Hkv} D{D} c{c} w{w} {dtype}")
    qd, k, v = inputs.decode_inputs(B, cache_len, Hkv * G, Hkv, D, dtype, seed=400 + idx, qk_scale=2.0)
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    o = to_np(dca.decode_varlen(qd.to(dev()), kc, v.to(dev()), kv, c, w))
    for b in range(B):
        Od, _ = oracle.dca_decode_ref(qd[b: b + 1], k[b: b + 1, : kv[b]], v[b: b + 1, : kv[b]], c, w)
        assert_close(o[b], Od[0], dtype, f"decode seq {b}")


@pytest.mark.parametrize("idx", range(N_CASES))
def test_sweep_paged_decode(idx):
    rng, dtype, D, Hkv, G, B, L = _draw("paged", idx)
    B = int(rng.integers(1, 6))
    c = int(rng.integers(2, 3000))
    w = int(rng.integers(0, c))
    P = int(rng.choice([16, 32, 48, 64]))
    kv = [int(rng.integers(1, 2500)) for _ in range(B)]
    log(f"[sweep paged] kv {kv} page {P} Hq{Hkv * G} Hkv{Hkv} D{D} c{c} w{w} {dtype}")
    qd, k, v = inputs.decode_inputs(B, max(kv), Hkv * G, Hkv, D, dtype, seed=500 + idx, qk_scale=2.0)
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    kp, table = to_pages(kc, kv, P, seed=idx)
    vp, _ = to_pages(v.to(dev()), kv, P, seed=idx)
    o = to_np(dca.decode_paged(qd.to(dev()), kp, vp, table, kv, c, w))
    for b in range(B):
        Od, _ = oracle.dca_decode_ref(qd[b: b + 1], k[b: b + 1, : kv[b]], v[b: b + 1, : kv[b]], c, w)
        assert_close(o[b], Od[0], dtype, f"paged decode seq {b}")


def _nan_tails(x, kv):
    x = x.clone()
    for b, n in enumerate(kv):
        x[b, n:] = float("nan")
    return x


@pytest.mark.parametrize("idx", range(N_CASES))
def test_sweep_selfextend_decode(idx):
    rng, dtype, D, Hkv, G, B, L = _draw("sedec", idx)
    B = int(rng.integers(1, 6))
    grp = int(rng.integers(1, 9))
    win = int(rng.choice([0, int(rng.integers(1, 1500)), 5000]))
    kv = [int(rng.integers(1, 2500)) for _ in range(B)]
    log(f"[sweep se decode] kv {kv} G{grp} W{win} Hq{Hkv * G} Hkv{Hkv} D{D} {dtype}")
    qd, k, v = inputs.decode_inputs(B, max(kv), Hkv * G, Hkv, D, dtype, seed=600 + idx, qk_scale=2.0)
    kg = k.to(dev())
    kp = _nan_tails(dca.rope_remap(kg, dca.DCA_MAP_PLAIN, 1, 0), kv)
    kq = _nan_tails(dca.rope_remap(kg, dca.DCA_MAP_SE_KEY_GROUPED, grp, win), kv)
    vd = _nan_tails(v.to(dev()), kv)
    od = dca.selfextend_decode(qd.to(dev()), kp, kq, vd, kv, grp, win)
    o = to_np(od)
    O, _ = oracle.selfextend_decode_ref(qd, k, v, kv, grp, win)
    for b in range(B):
        assert_close(o[b], O[b], dtype, f"selfextend decode seq {b}")
    # the same rows from page pools: the same bits
    P = int(rng.choice([16, 32, 48, 64]))
    pk, table = to_pages(kp, kv, P, seed=idx)
    pq, _ = to_pages(kq, kv, P, seed=idx)
    pv, _ = to_pages(vd, kv, P, seed=idx)
    assert torch.equal(dca.selfextend_decode_paged(qd.to(dev()), pk, pq, pv, table, kv, grp, win), od)


@pytest.mark.parametrize("idx", range(N_CASES))
def test_sweep_coarse_fine_decode(idx):
    rng, dtype, D, Hkv, G, B, L = _draw("cfdec", idx)
    B = int(rng.integers(1, 6))
    chunk = int(rng.integers(1, 700))
    train = int(rng.integers(1, 50))
    target = int(rng.integers(train, 8 * train + 1))
    kv = [int(rng.integers(1, 2500)) for _ in range(B)]
    log(f"[sweep cf decode] kv {kv} C{chunk} {train}->{target} Hq{Hkv * G} Hkv{Hkv} D{D} {dtype}")
    qd, k, v = inputs.decode_inputs(B, max(kv), Hkv * G, Hkv, D, dtype, seed=700 + idx, qk_scale=2.0)
    kg = k.to(dev())
    kp = _nan_tails(dca.rope_remap(kg, dca.DCA_MAP_PLAIN, 1, 0), kv)
    ks = _nan_tails(dca.coarse_fine_key_remap(kg, chunk, train, target), kv)
    vd = _nan_tails(v.to(dev()), kv)
    od = dca.coarse_fine_decode(qd.to(dev()), kp, ks, vd, kv, chunk, train, target)
    o = to_np(od)
    O, _ = oracle.coarse_fine_decode_ref(qd, k, v, kv, chunk, train, target)
    for b in range(B):
        assert_close(o[b], O[b], dtype, f"coarse/fine decode seq {b}")
    # the same rows from page pools: the same bits
    P = int(rng.choice([16, 32, 48, 64]))
    pk, table = to_pages(kp, kv, P, seed=idx)
    ps, _ = to_pages(ks, kv, P, seed=idx)
    pv, _ = to_pages(vd, kv, P, seed=idx)
    assert torch.equal(dca.coarse_fine_decode_paged(qd.to(dev()), pk, ps, pv, table, kv, chunk, train, target), od)
