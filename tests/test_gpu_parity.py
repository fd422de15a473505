"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars (written in each test): fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and
mean-abs <= 2e-3; dca_rope_remap within 1 bf16 ulp / 1e-6 for fp32.
Shapes span several tiles with ragged tails; the workload configurations
are checked on sampled rows the oracle evaluates one by one.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.dca_ref as ref
import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, want, dtype, what=""):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    mx, mean = float(err.max()), float(err.mean())
    if dtype == torch.float32:
        assert mx <= F32_TOL, f"{what}: max abs err {mx:.3e} > {F32_TOL}"
    else:
        assert mx <= BF16_MAX and mean <= BF16_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def bf16_lse_bar(scale, qn, kmax):
    """Worst-case bf16 LSE error, derived from the kernels' rounding.

    The rotated q and k are each rounded once to bf16 (relative error at most
    2^-8 per element), so a score q.k moves by at most
    ((1 + 2^-8)^2 - 1) * sum_d |q_d k_d| <= 2^-7 (1 + 2^-9) |q| |k| (rotations
    keep norms), times sm_scale; the LSE is 1-Lipschitz in the largest score
    change.  The kernels sum the normaliser from the fp32 probabilities and
    round them to bf16 only for the PV product; the 2^-8 term (what summing
    the rounded ones would move ln l by, -ln(1 - 2^-8) < 2^-8 (1 + 2^-8)) is
    kept as margin.  fp32 accumulation (dot products of 64-128 terms, a few
    thousand tile sums) adds well under 1e-5 relative; 1e-4 absolute covers
    it."""
    return 2.0 ** -7 * (1 + 2.0 ** -8) * scale * qn * kmax + 2.0 ** -8 * (1 + 2.0 ** -7) + 1e-4


def lse_bound_prefill(q, k, dtype):
    """LSE bar: fp32 1e-4; bf16 bf16_lse_bar(scale, |q_i|, max_{j<=i} |k_j|)."""
    if dtype == torch.float32:
        return F32_TOL
    qn = np.linalg.norm(np.asarray(q.float(), np.float64), axis=-1)          # [B, L, Hq]
    kn = np.linalg.norm(np.asarray(k.float(), np.float64), axis=-1)          # [B, L, Hkv]
    kmax = np.maximum.accumulate(kn, axis=1)
    G = q.shape[2] // k.shape[2]
    kmax = np.repeat(kmax, G, axis=2)
    scale = 1.0 / math.sqrt(q.shape[-1])
    return bf16_lse_bar(scale, qn, kmax).transpose(0, 2, 1)                    # [B, Hq, L]


def lse_bound_decode(q, k, dtype):
    if dtype == torch.float32:
        return F32_TOL
    qn = np.linalg.norm(np.asarray(q.float(), np.float64), axis=-1)          # [B, Hq]
    kmax = np.linalg.norm(np.asarray(k.float(), np.float64), axis=-1).max(axis=1)  # [B, Hkv]
    kmax = np.repeat(kmax, q.shape[1] // k.shape[2], axis=1)
    return bf16_lse_bar(1.0 / math.sqrt(q.shape[-1]), qn, kmax)


def bf16_ulp(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


# ---------------------------------------------------------------- remap -----
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("pos0", [0, 777])
def test_rope_remap_all_maps(dtype, D, pos0):
    c, w = 128, 32
    x = inputs.prefill_inputs(2, 301, 3, 3, D, dtype, seed=5, qk_scale=1.0)[0]
    xg = x.to(dev())
    for m in range(5):
        got = to_np(dca.rope_remap(xg, m, c, w, 1e4, pos0))
        want = oracle.rope_remap_ref(x, pos0, m, c, w, 1e4)
        err = np.abs(got - want)
        if dtype == torch.float32:
            assert err.max() <= 1e-6, (m, err.max())
        else:
            assert np.all(err <= bf16_ulp(want) + 1e-30), (m, err.max())
    # in place
    y = xg.clone()
    dca.rope_remap(y, dca.DCA_MAP_KEY, c, w, 1e4, pos0, out=y)
    assert torch.equal(y, dca.rope_remap(xg, dca.DCA_MAP_KEY, c, w, 1e4, pos0))


def test_rope_remap_rounds_once():
    # The bf16 remap (and the prepare pass, bit-identical to it) returns the
    # fp64 rotation rounded once to bf16, so it lies within half a bf16 ulp of
    # the oracle's rotation, up to the fp64 differences between the two angle
    # evaluations (1e-11 of the pair's magnitude covers them).  Rounding
    # through fp32 without the midpoint repair would exceed half an ulp on
    # the values whose fp32 rounding lands on a bf16 midpoint; the input is
    # large enough to hold many of those.
    c, w = 4096, 1024
    x = inputs.prefill_inputs(4, 2048, 8, 8, 128, torch.bfloat16, seed=21, qk_scale=1.0)[0]
    got = to_np(dca.rope_remap(x.to(dev()), dca.DCA_MAP_KEY, c, w, 1e4))
    want = oracle.rope_remap_ref(x, 0, oracle.MAP_KEY, c, w, 1e4)
    xf = to_np(x)
    m = np.abs(xf[..., :64]) + np.abs(xf[..., 64:])
    tol = 0.5 * bf16_ulp(want) + 1e-11 * np.concatenate([m, m], axis=-1)
    err = np.abs(got - want)
    assert np.all(err <= tol), (err - tol).max()
    mid = (want.astype(np.float32).view(np.uint32) & 0xFFFF) == 0x8000
    assert np.count_nonzero(mid) >= 20, np.count_nonzero(mid)


@pytest.mark.parametrize("B,L,H", [(17, 5, 64), (1, 1, 1), (3, 9, 2), (2, 130, 40)])
def test_rope_remap_shapes(B, L, H):
    # token counts that are not multiples of the 4 tokens a workgroup takes,
    # head counts whose rows exceed one pass of the workgroup, batch > 16
    for dtype, D in ((torch.bfloat16, 128), (torch.float32, 64)):
        x = inputs.prefill_inputs(B, L, H, H, D, dtype, seed=15, qk_scale=1.0)[0]
        got = to_np(dca.rope_remap(x.to(dev()), dca.DCA_MAP_KEY, 96, 32, 1e4, 41))
        want = oracle.rope_remap_ref(x, 41, oracle.MAP_KEY, 96, 32, 1e4)
        err = np.abs(got - want)
        if dtype == torch.float32:
            assert err.max() <= 1e-6, (B, L, H, err.max())
        else:
            assert np.all(err <= bf16_ulp(want) + 1e-30), (B, L, H, err.max())


# ----------------------------------------------------- prefill, small -------
SMALL = [
    # name, B, L, Hq, Hkv, D, c, w, dtype, qk_scale
    ("tiny_f32_config", 1, 512, 1, 1, 64, 128, 32, torch.float32, None),
    ("tiny_f32_discriminating", 1, 512, 1, 1, 64, 128, 32, torch.float32, 2.0),
    ("f32_gqa_ragged_d128", 2, 333, 4, 2, 128, 64, 16, torch.float32, 2.0),
    ("f32_w0_s_small", 1, 150, 2, 1, 64, 24, 0, torch.float32, 2.0),
    ("bf16_fast_path", 2, 700, 4, 2, 128, 256, 64, torch.bfloat16, 2.0),
    ("bf16_straddle_s96_d64", 1, 512, 2, 1, 64, 128, 32, torch.bfloat16, 2.0),
    ("bf16_straddle_s96_d128", 1, 600, 2, 2, 128, 128, 32, torch.bfloat16, 2.0),
    ("bf16_many_chunks_s40", 1, 333, 2, 1, 128, 56, 16, torch.bfloat16, 2.0),
    ("bf16_s1", 1, 130, 1, 1, 64, 1, 0, torch.bfloat16, 2.0),
    ("bf16_w_gt_s", 1, 400, 2, 1, 128, 100, 70, torch.bfloat16, 2.0),
    ("bf16_config_scale", 1, 1000, 8, 1, 128, 512, 128, torch.bfloat16, None),
    ("bf16_L1", 1, 1, 2, 2, 128, 128, 32, torch.bfloat16, 2.0),
    ("bf16_L63", 3, 63, 2, 1, 64, 128, 32, torch.bfloat16, 2.0),
    ("bf16_L129", 1, 129, 4, 4, 128, 128, 64, torch.bfloat16, 2.0),
    # chunk sizes that are multiples of 64 (the two-group kernel), ragged lengths
    ("bf16_s64_d64_ragged", 2, 777, 4, 2, 64, 96, 32, torch.bfloat16, 2.0),
    ("bf16_s128_w0_gqa", 1, 1000, 8, 2, 128, 128, 0, torch.bfloat16, 2.0),
    ("bf16_s64_L1", 1, 1, 2, 1, 128, 64, 0, torch.bfloat16, 2.0),
    ("bf16_s64_L300", 1, 300, 2, 2, 128, 100, 36, torch.bfloat16, 2.0),
    ("bf16_s256_L257", 3, 257, 2, 1, 64, 320, 64, torch.bfloat16, 2.0),
    # KV head counts that leave the prepare pass's last 8-head group partly
    # empty: one group (6, 5, 3 heads) and a full group plus a partial one (12)
    ("bf16_hkv6_gqa2", 1, 400, 12, 6, 128, 192, 64, torch.bfloat16, 2.0),
    ("bf16_hkv5_mha_d64", 2, 250, 5, 5, 64, 128, 0, torch.bfloat16, 2.0),
    ("bf16_hkv3_s_straddle", 1, 300, 6, 3, 128, 100, 4, torch.bfloat16, 2.0),
    ("bf16_hkv12_two_groups", 2, 333, 24, 12, 128, 192, 64, torch.bfloat16, 2.0),
    ("bf16_hkv10_d64_two_groups", 1, 190, 10, 10, 64, 128, 32, torch.bfloat16, 2.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_prefill_full_parity(case):
    name, B, L, Hq, Hkv, D, c, w, dtype, a = case
    log(f"[prefill] {name}")
    q, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, dtype, seed=100, qk_scale=a)
    o, lse, krot = dca.prefill(q.to(dev()), k.to(dev()), v.to(dev()), c, w, 1e4,
                               return_lse=True, return_k_rot=True)
    torch.cuda.synchronize()
    O, LSE = oracle.dca_prefill_ref(q, k, v, c, w, 1e4)
    assert_close(to_np(o), O, dtype, name)
    assert np.all(np.abs(to_np(lse) - LSE) <= lse_bound_prefill(q, k, dtype))
    # rotated keys handed back as a decode cache
    Kr = oracle.rope_remap_ref(k, 0, oracle.MAP_KEY, c, w, 1e4)
    err = np.abs(to_np(krot) - Kr)
    if dtype == torch.float32:
        assert err.max() <= 1e-6
    else:
        assert np.all(err <= bf16_ulp(Kr) + 1e-30)
    # the prepare pass and dca_rope_remap round every key alike
    assert torch.equal(krot, dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w, 1e4))


def _mutant_succ_as_inter(monkeypatch):
    good = ref.query_positions

    def succ_as_inter(i, c, w):
        a_, b_, e_ = good(i, c, w)
        return a_, e_, e_
    monkeypatch.setattr(ref, "query_positions", succ_as_inter)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_separation_ratio(dtype, monkeypatch):
    """A wrong successive map must be >= 10x further from the oracle than the GPU is."""
    B, L, Hq, Hkv, D, c, w = 1, 512, 2, 1, 64, 128, 32
    q, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, dtype, seed=7, qk_scale=2.0)
    o = to_np(dca.prefill(q.to(dev()), k.to(dev()), v.to(dev()), c, w, 1e4))
    O, _ = oracle.dca_prefill_ref(q, k, v, c, w, 1e4)
    _mutant_succ_as_inter(monkeypatch)
    Ow, _ = oracle.dca_prefill_ref(q, k, v, c, w, 1e4)
    ratio = np.linalg.norm(Ow - O) / max(np.linalg.norm(o - O), 1e-30)
    log(f"separation ratio {dtype}: {ratio:.1f}")
    assert ratio >= 10.0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", ["intra", "succ_exact", "succ_saturated", "inter", "inter_far"])
def test_prefill_planted_keys(dtype, case):
    from test_oracle_pins import PLANTED, planted_case
    c, w, i, jstar = PLANTED[case]
    D = 64
    q, k, v, want = planted_case(c, w, i, jstar, D=D, seed=3)
    # pad the sequence past i so the row sits inside a longer causal prefill
    L = i + 70
    pad = lambda x: np.concatenate([x, np.random.default_rng(1).standard_normal((1, 70, 1, D)) * 0.1], 1)
    qt, kt, vt = (torch.from_numpy(pad(x)).to(dtype) for x in (q, k, v))
    o = to_np(dca.prefill(qt.to(dev()), kt.to(dev()), vt.to(dev()), c, w, 1e4))
    O, _ = oracle.dca_prefill_ref(qt, kt, vt, c, w, 1e4, rows=[i])
    assert_close(o[:, i], O[:, 0], dtype, case)
    if dtype == torch.float32:   # inputs exact: the closed form holds too
        assert np.abs(o[0, i, 0] - want).max() <= F32_TOL


# Chunk size a multiple of 64 (the two-group kernel) and a planted logit of 12:
# the planted probability is about 2^17 times the others, far past the
# per-lane sum that forces the running max to move at a later key tile.
PLANTED_RESCALE = {
    "succ_exact_s128": (192, 64, 300, 200),   # rho 1, r(i) = 44 < w
    "inter_s128": (192, 64, 700, 150),        # rho 4
}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", sorted(PLANTED_RESCALE))
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_planted_rescale(dtype, case, D):
    from test_oracle_pins import planted_case
    c, w, i, jstar = PLANTED_RESCALE[case]
    q, k, v, want = planted_case(c, w, i, jstar, D=D, seed=4, target_logit=12.0)
    L = i + 70
    pad = lambda x: np.concatenate([x, np.random.default_rng(2).standard_normal((1, 70, 1, D)) * 0.1], 1)
    qt, kt, vt = (torch.from_numpy(pad(x)).to(dtype) for x in (q, k, v))
    o, lse = dca.prefill(qt.to(dev()), kt.to(dev()), vt.to(dev()), c, w, 1e4, return_lse=True)
    O, LSE = oracle.dca_prefill_ref(qt, kt, vt, c, w, 1e4, rows=[i])
    assert_close(to_np(o)[:, i], O[:, 0], dtype, case)
    bound = lse_bound_prefill(qt, kt, dtype)
    bound = bound if np.isscalar(bound) else bound[0, 0, i]
    assert abs(to_np(lse)[0, 0, i] - LSE[0, 0, 0]) <= bound
    if dtype == torch.float32:
        assert np.abs(to_np(o)[0, i, 0] - want).max() <= F32_TOL


def test_prefill_deterministic_and_causal():
    B, L, Hq, Hkv, D, c, w = 1, 777, 4, 1, 128, 256, 64
    q, k, v = (x.to(dev()) for x in inputs.prefill_inputs(B, L, Hq, Hkv, D, "bf16", seed=9, qk_scale=2.0))
    o1 = dca.prefill(q, k, v, c, w)
    o2 = dca.prefill(q, k, v, c, w)
    assert torch.equal(o1, o2)
    k2, v2 = k.clone(), v.clone()
    k2[:, 400:] = 3.0
    v2[:, 400:] = -2.0
    o3 = dca.prefill(q, k2, v2, c, w)
    assert torch.equal(o1[:, :400], o3[:, :400])


def test_prefill_constant_v_gives_constant_output():
    q, k, v = (x.to(dev()) for x in inputs.prefill_inputs(1, 500, 2, 1, 128, "bf16", seed=2, qk_scale=3.0))
    o = dca.prefill(q, k, torch.ones_like(v), 128, 32)
    assert (o.float() - 1.0).abs().max().item() <= 2.0 ** -7


# ---------------------------------------------------------------- decode ----
DECODE = [
    # name, B, kv_len, Hq, Hkv, D, c, w, dtype, qk_scale
    ("bf16_gqa8", 2, 3000, 16, 2, 128, 512, 128, torch.bfloat16, 2.0),
    ("bf16_straddle_s96", 2, 1001, 8, 8, 64, 128, 32, torch.bfloat16, 2.0),
    ("bf16_mqa_g64", 1, 777, 64, 1, 128, 256, 64, torch.bfloat16, 2.0),
    ("bf16_kv1", 2, 1, 4, 2, 128, 128, 32, torch.bfloat16, 2.0),
    ("bf16_kv31", 1, 31, 4, 1, 64, 16, 4, torch.bfloat16, 2.0),
    ("bf16_config_scale", 2, 5000, 64, 8, 128, 4096, 1024, torch.bfloat16, None),
    ("f32_gqa", 2, 2000, 8, 2, 128, 256, 64, torch.float32, 2.0),
    ("f32_straddle", 1, 999, 4, 4, 64, 128, 32, torch.float32, 2.0),
]


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_decode_parity(case):
    name, B, kv_len, Hq, Hkv, D, c, w, dtype, a = case
    log(f"[decode] {name}")
    q, k, v = inputs.decode_inputs(B, kv_len, Hq, Hkv, D, dtype, seed=31, qk_scale=a)
    kg = k.to(dev())
    kc = dca.rope_remap(kg, dca.DCA_MAP_KEY, c, w, 1e4, 0)
    o, lse = dca.decode(q.to(dev()), kc, v.to(dev()), c, w, 1e4, return_lse=True)
    torch.cuda.synchronize()
    O, LSE = oracle.dca_decode_ref(q, k, v, c, w, 1e4)
    assert_close(to_np(o), O, dtype, name)
    assert np.all(np.abs(to_np(lse) - LSE) <= lse_bound_decode(q, k, dtype))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_equals_last_prefill_row(dtype):
    B, L, Hq, Hkv, D, c, w = 2, 1500, 8, 2, 128, 512, 128
    q, k, v = (x.to(dev()) for x in inputs.prefill_inputs(B, L, Hq, Hkv, D, dtype, seed=4, qk_scale=2.0))
    o, kr = dca.prefill(q, k, v, c, w, return_k_rot=True)
    od = dca.decode(q[:, L - 1].contiguous(), kr, v, c, w)
    assert_close(to_np(od), to_np(o[:, L - 1]), dtype, "decode vs prefill row")


def test_decode_planted_keys_bf16():
    from test_oracle_pins import PLANTED, planted_case
    for case in ("intra", "succ_saturated", "inter_far"):
        c, w, i, jstar = PLANTED[case]
        q, k, v, _ = planted_case(c, w, i, jstar, D=64, seed=5)
        qt, kt, vt = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
        kc = dca.rope_remap(kt.to(dev()), dca.DCA_MAP_KEY, c, w)
        od = dca.decode(qt[:, i].contiguous().to(dev()), kc, vt.to(dev()), c, w)
        Od, _ = oracle.dca_decode_ref(qt[:, i], kt, vt, c, w)
        assert_close(to_np(od), Od, torch.bfloat16, case)
