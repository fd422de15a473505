"""GPU parity of decode under the SelfExtend and coarse / fine maps, and of the
coarse-scaled key remap, through the C ABI against the fp64 oracle.

Definition: the new token of sequence b is row kv_len[b] - 1 of the map's
prefill over its first kv_len[b] keys ("LLM Maybe LongLM: Self-Extend LLM
Context Window Without Tuning", abstract; "Dual-Chunk Attention:
Training-Free 100k+ Context Guide", "Inter-Chunk Attention" and "Successive
Chunk Smoothing").  The two key caches hold every row of the sequence; rows
past each sequence's length are NaN, so a read of them would show.  Bars:
fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and mean-abs <= 2e-3; the remap
within 1 bf16 ulp (fp32: 1e-6).
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs
from test_gpu_parity import assert_close, bf16_ulp, dev, log, to_np

pytestmark = pytest.mark.gpu


def nan_tails(x, kv):
    x = x.clone()
    for b, n in enumerate(kv):
        x[b, n:] = float("nan")
    return x


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("C,train,target,pos0", [(64, 4, 32, 0), (100, 3, 7, 333), (7, 1, 1, 5)])
def test_coarse_fine_key_remap(dtype, C, train, target, pos0):
    x = inputs.prefill_inputs(2, 300, 3, 3, 128, dtype, seed=7, qk_scale=1.0)[0]
    got = to_np(dca.coarse_fine_key_remap(x.to(dev()), C, train, target, 1e4, pos0))
    want = oracle.coarse_fine_key_remap_ref(x, pos0, C, train, target, 1e4)
    err = np.abs(got - want)
    if dtype == torch.float32:
        assert err.max() <= 1e-6, err.max()
    else:
        assert np.all(err <= bf16_ulp(want) + 1e-30), err.max()


SE_DEC = [
    # name, kv list, Hq, Hkv, D, G, W, dtype
    ("bf16_g4_w100", [1, 50, 99, 100, 101, 700], 8, 2, 128, 4, 100, torch.bfloat16),
    ("bf16_w0_all_grouped", [33, 400], 4, 1, 64, 3, 0, torch.bfloat16),
    ("bf16_window_covers", [5, 300], 4, 4, 128, 8, 10 ** 6, torch.bfloat16),
    ("bf16_g1", [77, 1000], 16, 2, 128, 1, 37, torch.bfloat16),
    ("bf16_long_ragged", [4097, 2500, 9000], 64, 8, 128, 8, 1024, torch.bfloat16),
    ("f32_g5_w33", [1, 34, 35, 600], 4, 2, 64, 5, 33, torch.float32),
    ("f32_w0", [20, 257], 2, 1, 128, 2, 0, torch.float32),
]


@pytest.mark.parametrize("case", SE_DEC, ids=[c[0] for c in SE_DEC])
def test_selfextend_decode_matches_oracle(case):
    name, kv, Hq, Hkv, D, G, W, dtype = case
    log(f"[se decode] {name}")
    B, L = len(kv), max(kv)
    qd, k, v = inputs.decode_inputs(B, L, Hq, Hkv, D, dtype, seed=600, qk_scale=2.0)
    kg = k.to(dev())
    k_plain = nan_tails(dca.rope_remap(kg, dca.DCA_MAP_PLAIN, 1, 0), kv)
    k_grp = nan_tails(dca.rope_remap(kg, dca.DCA_MAP_SE_KEY_GROUPED, G, min(W, 1 << 30)), kv)
    vc = nan_tails(v.to(dev()), kv)
    o = to_np(dca.selfextend_decode(qd.to(dev()), k_plain, k_grp, vc, kv, G, W))
    O, _ = oracle.selfextend_decode_ref(qd, k, v, kv, G, W)
    for b in range(B):
        assert_close(o[b], O[b], dtype, f"{name} seq {b}")


CF_DEC = [
    # name, kv list, Hq, Hkv, D, C, train, target, dtype
    ("bf16_c64_k8", [1, 64, 65, 128, 129, 700], 8, 2, 128, 64, 1, 8, torch.bfloat16),
    ("bf16_c100_frac", [99, 100, 201, 1000], 4, 1, 64, 100, 3, 7, torch.bfloat16),
    ("bf16_guide_params", [600, 2048, 5000], 16, 2, 128, 512, 4096, 32768, torch.bfloat16),
    ("bf16_kappa1", [300, 777], 4, 4, 128, 50, 5, 5, torch.bfloat16),
    ("f32_c13", [1, 13, 14, 27, 400], 4, 2, 64, 13, 2, 9, torch.float32),
]


@pytest.mark.parametrize("case", CF_DEC, ids=[c[0] for c in CF_DEC])
def test_coarse_fine_decode_matches_oracle(case):
    name, kv, Hq, Hkv, D, C, tr, tg, dtype = case
    log(f"[cf decode] {name}")
    B, L = len(kv), max(kv)
    qd, k, v = inputs.decode_inputs(B, L, Hq, Hkv, D, dtype, seed=601, qk_scale=2.0)
    kg = k.to(dev())
    k_plain = nan_tails(dca.rope_remap(kg, dca.DCA_MAP_PLAIN, 1, 0), kv)
    k_sc = nan_tails(dca.coarse_fine_key_remap(kg, C, tr, tg), kv)
    vc = nan_tails(v.to(dev()), kv)
    o = to_np(dca.coarse_fine_decode(qd.to(dev()), k_plain, k_sc, vc, kv, C, tr, tg))
    O, _ = oracle.coarse_fine_decode_ref(qd, k, v, kv, C, tr, tg)
    for b in range(B):
        assert_close(o[b], O[b], dtype, f"{name} seq {b}")


@pytest.mark.parametrize("which", ["selfextend", "coarse_fine"])
def test_map_decode_equals_last_prefill_row(which):
    L, Hq, Hkv, D = 1000, 8, 2, 128
    q, k, v = (x.to(dev()) for x in inputs.prefill_inputs(1, L, Hq, Hkv, D, "bf16", seed=602, qk_scale=2.0))
    plain = dca.rope_remap(k, dca.DCA_MAP_PLAIN, 1, 0)
    if which == "selfextend":
        full = dca.selfextend_prefill(q, k, v, 4, 128)
        dec = dca.selfextend_decode(q[:, -1].contiguous(), plain, dca.rope_remap(k, dca.DCA_MAP_SE_KEY_GROUPED, 4, 128),
                                    v, [L], 4, 128)
    else:
        full = dca.coarse_fine_prefill(q, k, v, 128, 1, 8)
        dec = dca.coarse_fine_decode(q[:, -1].contiguous(), plain, dca.coarse_fine_key_remap(k, 128, 1, 8), v, [L],
                                     128, 1, 8)
    assert (full[:, -1].float() - dec.float()).abs().max() <= 2e-2


def test_map_decode_100k_workload():
    # decode_100k's shape with ragged lengths: SelfExtend (G 8, W 1024) and the
    # guide's coarse / fine parameters (C 512, 4096 -> 32768), sampled sequences.
    P = inputs.WORKLOADS["decode_100k"]
    B, kvmax, Hq, Hkv, D = (P[x] for x in ("B", "kv_len", "Hq", "Hkv", "D"))
    kv = [int(x) for x in np.linspace(kvmax // 2, kvmax, B)]
    qd, k, v = inputs.decode_inputs(B, kvmax, Hq, Hkv, D, "bf16", seed=P["seed"])
    kg = k.to(dev())
    plain = dca.rope_remap(kg, dca.DCA_MAP_PLAIN, 1, 0)
    second = dca.rope_remap(kg, dca.DCA_MAP_SE_KEY_GROUPED, 8, 1024)
    vc = v.to(dev())
    o_se = to_np(dca.selfextend_decode(qd.to(dev()), plain, second, vc, kv, 8, 1024))
    dca.coarse_fine_key_remap(kg, 512, 4096, 32768, out=second)
    del kg
    o_cf = to_np(dca.coarse_fine_decode(qd.to(dev()), plain, second, vc, kv, 512, 4096, 32768))
    for b in (0, 15):
        sl = slice(b, b + 1)
        Os, _ = oracle.selfextend_decode_ref(qd[sl], k[sl], v[sl], kv[b: b + 1], 8, 1024)
        mx, _ = assert_close(o_se[b], Os[0], torch.bfloat16, f"selfextend decode seq {b}")
        Oc, _ = oracle.coarse_fine_decode_ref(qd[sl], k[sl], v[sl], kv[b: b + 1], 512, 4096, 32768)
        mx2, _ = assert_close(o_cf[b], Oc[0], torch.bfloat16, f"coarse/fine decode seq {b}")
        log(f"  seq {b} (kv_len {kv[b]}): selfextend max abs {mx:.3e}, coarse/fine max abs {mx2:.3e}")
