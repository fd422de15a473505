"""GPU parity of SelfExtend grouped / neighbor attention (through the C ABI)
against the fp64 oracle.

Source: "LLM Maybe LongLM: Self-Extend LLM Context Window Without Tuning"
(abstract).  Bars: fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and mean-abs
<= 2e-3; LSE within the bf16 rounding bound; remap within 1 bf16 ulp / 1e-6.
Cases cover the reductions to ordinary RoPE (G = 1, W >= L), W = 0, windows
that are and are not multiples of the 64-key tile, ragged lengths, GQA and
both head dims; the 32k workload is checked on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs
from test_gpu_parity import (BF16_MAX, F32_TOL, assert_close, bf16_ulp, dev, log,
                             lse_bound_prefill, to_np)
from test_selfextend_pins import SE_PLANTED, se_planted_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,W,pos0", [(4, 100, 0), (3, 7, 555), (1, 0, 9)])
def test_rope_remap_grouped_maps(dtype, D, G, W, pos0):
    x = inputs.prefill_inputs(2, 301, 3, 3, D, dtype, seed=6, qk_scale=1.0)[0]
    xg = x.to(dev())
    for m in (dca.DCA_MAP_SE_KEY_GROUPED, dca.DCA_MAP_SE_Q_GROUPED):
        got = to_np(dca.rope_remap(xg, m, G, W, 1e4, pos0))
        want = oracle.se_rope_remap_ref(x, pos0, m, G, W, 1e4)
        err = np.abs(got - want)
        if dtype == torch.float32:
            assert err.max() <= 1e-6, (m, err.max())
        else:
            assert np.all(err <= bf16_ulp(want) + 1e-30), (m, err.max())


SE_SMALL = [
    # name, B, L, Hq, Hkv, D, G, W, dtype, qk_scale
    ("f32_g4_w100", 1, 333, 2, 1, 64, 4, 100, torch.float32, 2.0),
    ("f32_g8_w64_d128_gqa", 2, 300, 4, 2, 128, 8, 64, torch.float32, 2.0),
    ("f32_g1_plain", 1, 200, 2, 2, 64, 1, 37, torch.float32, 2.0),
    ("f32_w0_all_grouped", 1, 150, 1, 1, 64, 3, 0, torch.float32, 2.0),
    ("f32_window_covers", 1, 180, 1, 1, 128, 5, 500, torch.float32, 2.0),
    ("bf16_g4_w100", 1, 700, 4, 2, 128, 4, 100, torch.bfloat16, 2.0),
    ("bf16_g8_w256_d64", 2, 1000, 4, 1, 64, 8, 256, torch.bfloat16, 2.0),
    ("bf16_g2_w1", 1, 517, 2, 2, 128, 2, 1, torch.bfloat16, 2.0),
    ("bf16_w0", 1, 400, 2, 1, 64, 4, 0, torch.bfloat16, 2.0),
    ("bf16_g1", 1, 600, 2, 1, 128, 1, 70, torch.bfloat16, 2.0),
    ("bf16_window_covers", 1, 300, 2, 2, 128, 16, 4096, torch.bfloat16, 2.0),
    ("bf16_config_scale", 1, 1500, 8, 2, 128, 8, 512, torch.bfloat16, None),
    ("bf16_L1", 1, 1, 2, 1, 128, 4, 16, torch.bfloat16, 2.0),
    ("bf16_L65_w64", 2, 65, 2, 2, 64, 4, 64, torch.bfloat16, 2.0),
    ("bf16_g7_w33_ragged", 3, 259, 2, 1, 128, 7, 33, torch.bfloat16, 2.0),
    ("bf16_hkv6_d64", 1, 300, 6, 6, 64, 4, 100, torch.bfloat16, 2.0),
    ("bf16_hkv9_two_groups", 1, 270, 9, 9, 128, 4, 64, torch.bfloat16, 2.0),
]


@pytest.mark.parametrize("case", SE_SMALL, ids=[c[0] for c in SE_SMALL])
def test_selfextend_full_parity(case):
    name, B, L, Hq, Hkv, D, G, W, dtype, a = case
    log(f"[selfextend] {name}")
    q, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, dtype, seed=200, qk_scale=a)
    o, lse = dca.selfextend_prefill(q.to(dev()), k.to(dev()), v.to(dev()), G, W, 1e4, return_lse=True)
    O, LSE = oracle.selfextend_prefill_ref(q, k, v, G, W, 1e4)
    mx, mean = assert_close(to_np(o), O, dtype, name)
    lerr = np.abs(to_np(lse) - LSE)
    assert np.all(lerr <= lse_bound_prefill(q, k, dtype)), (name, lerr.max())
    log(f"  O max {mx:.2e} mean {mean:.2e}  LSE max {lerr.max():.2e}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", sorted(SE_PLANTED))
def test_selfextend_planted_keys(dtype, case):
    G, W, i, jstar = SE_PLANTED[case]
    D = 64
    q, k, v, want = se_planted_case(G, W, i, jstar, D=D, seed=3)
    L = i + 70
    pad = lambda x: np.concatenate([x, np.random.default_rng(1).standard_normal((1, 70, 1, D)) * 0.1], 1)
    qt, kt, vt = (torch.from_numpy(pad(x)).to(dtype) for x in (q, k, v))
    o = to_np(dca.selfextend_prefill(qt.to(dev()), kt.to(dev()), vt.to(dev()), G, W, 1e4))
    O, _ = oracle.selfextend_prefill_ref(qt, kt, vt, G, W, 1e4, rows=[i])
    assert_close(o[:, i], O[:, 0], dtype, case)
    if dtype == torch.float32:
        assert np.abs(o[0, i, 0] - want).max() <= F32_TOL


def test_selfextend_group_swap_invariance():
    # Two keys of one group, both grouped with respect to row i, carry one key
    # position: swapping their K/V rows leaves row i unchanged (up to the order
    # of the sums); two keys of different groups do not.
    G, W, L, D = 4, 64, 300, 64
    q, k, v = inputs.prefill_inputs(1, L, 1, 1, D, torch.float32, seed=31, qk_scale=2.0)
    i, j1, j2, j3 = 299, 100, 103, 104
    run = lambda kk, vv: to_np(dca.selfextend_prefill(q.to(dev()), kk.to(dev()), vv.to(dev()), G, W))[0, i, 0]
    base = run(k, v)
    k2, v2 = k.clone(), v.clone()
    k2[:, [j1, j2]] = k[:, [j2, j1]]
    v2[:, [j1, j2]] = v[:, [j2, j1]]
    assert np.abs(run(k2, v2) - base).max() <= 1e-6
    k3, v3 = k.clone(), v.clone()
    k3[:, [j1, j3]] = k[:, [j3, j1]]
    v3[:, [j1, j3]] = v[:, [j3, j1]]
    assert np.abs(run(k3, v3) - base).max() > 1e-4


def test_selfextend_deterministic_and_causal():
    # Rows before a cut do not depend on the keys / values after it.  A wave
    # owns 32 rows and takes its exact-rescale decision for all of them, so a
    # row sharing a wave with changed rows may be computed through the exact
    # path instead (the same value up to rounding); rows of other waves are
    # bit-identical.
    q, k, v = (x.to(dev()) for x in inputs.prefill_inputs(1, 777, 4, 1, 128, "bf16", seed=9, qk_scale=2.0))
    o1 = dca.selfextend_prefill(q, k, v, 8, 128)
    assert torch.equal(o1, dca.selfextend_prefill(q, k, v, 8, 128))
    for cut in (512, 500):
        k2, v2 = k.clone(), v.clone()
        k2[:, cut:] = 3.0
        v2[:, cut:] = -2.0
        o2 = dca.selfextend_prefill(q, k2, v2, 8, 128)
        whole = cut // 32 * 32   # rows in waves wholly before the cut
        assert torch.equal(o1[:, :whole], o2[:, :whole]), cut
        if whole < cut:
            assert (o1[:, whole:cut].float() - o2[:, whole:cut].float()).abs().max() <= 2e-2, cut


def test_selfextend_32k_workload_sampled_rows():
    P = inputs.WORKLOADS["selfextend_70b_32k"]
    B, L, Hq, Hkv, D, G, W = (P[x] for x in ("B", "L", "Hq", "Hkv", "D", "group", "window"))
    log(f"[selfextend] workload L={L} G={G} W={W}")
    q, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, P["dtype"], seed=P["seed"])
    o, lse = dca.selfextend_prefill(q.to(dev()), k.to(dev()), v.to(dev()), G, W, P["base"], return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = sorted({0, 1, 63, 64, W - 1, W, W + 1, W + 63, W + 64, 2 * W, L - 2, L - 1}
                  | set(rng.integers(0, L, 12).tolist()))
    heads = [0, 7, 8, 33, 63]
    O, LSE = oracle.selfextend_prefill_ref(q, k, v, G, W, P["base"], rows=rows, heads=heads)
    got = to_np(o[:, rows][:, :, heads])
    mx, mean = assert_close(got, O, torch.bfloat16, "selfextend_70b_32k")
    lerr = np.abs(to_np(lse[:, heads][:, :, rows]) - LSE)
    assert lerr.max() <= BF16_MAX, lerr.max()
    log(f"  selfextend_70b_32k O: max abs {mx:.3e}, mean abs {mean:.3e}; LSE max {lerr.max():.2e}")
