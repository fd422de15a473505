"""GPU parity of the DCA guide's coarse / fine distance map (through the C ABI)
against the fp64 oracle.

Source: "Dual-Chunk Attention: Training-Free 100k+ Context Guide", sections
"Inter-Chunk Attention" and "Successive Chunk Smoothing".  Bars: fp32 max-abs
<= 1e-4; bf16 max-abs <= 2e-2 and mean-abs <= 2e-3; LSE within the bf16
rounding bound.  Cases include kappa = 1 (plain RoPE), chunk / kappa ratios
that are not integers, the guide's own parameters and, for bf16, the chunk
sizes that are multiples of the 64-key tile (others are rejected).
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs
from test_coarse_fine_pins import cf_planted_case
from test_gpu_parity import F32_TOL, assert_close, dev, log, lse_bound_prefill, to_np

pytestmark = pytest.mark.gpu

CF_SMALL = [
    # name, B, L, Hq, Hkv, D, C, train_len, target_len, dtype, qk_scale
    ("f32_c16_k2", 1, 150, 2, 1, 64, 16, 4, 8, torch.float32, 2.0),
    ("f32_c12_frac", 1, 100, 2, 2, 128, 12, 3, 7, torch.float32, 2.0),
    ("f32_kappa1", 1, 120, 1, 1, 64, 32, 5, 5, torch.float32, 2.0),
    ("bf16_c64_k8_gqa", 1, 700, 8, 2, 128, 64, 1, 8, torch.bfloat16, 2.0),
    ("bf16_c128_frac_d64", 2, 1000, 4, 1, 64, 128, 2, 5, torch.bfloat16, 2.0),
    ("bf16_kappa1", 1, 300, 2, 2, 128, 64, 7, 7, torch.bfloat16, 2.0),
    ("bf16_guide_params", 1, 2000, 4, 1, 128, 512, 4096, 32768, torch.bfloat16, 2.0),
    ("bf16_L65_ragged", 3, 65, 2, 1, 128, 64, 3, 10, torch.bfloat16, 2.0),
    ("bf16_config_scale", 1, 1500, 8, 1, 128, 256, 1, 4, torch.bfloat16, None),
    # workgroups (256 rows) spanning chunks whose relation to one key tile
    # differs (rows past L included): the staged key rotation must not follow
    # any one wave's relation
    ("bf16_c64_l128_mixed_workgroup", 1, 128, 1, 1, 128, 64, 1, 8, torch.bfloat16, 2.0),
    ("bf16_c128_three_relations_one_wg", 1, 600, 2, 1, 64, 128, 1, 8, torch.bfloat16, 2.0),
    # KV head counts that fill the prepare pass's 8-head group partly (5), or
    # one group and part of a second (11)
    ("bf16_hkv5", 1, 300, 10, 5, 128, 64, 2, 9, torch.bfloat16, 2.0),
    ("bf16_hkv11_two_groups_d64", 1, 260, 11, 11, 64, 64, 2, 9, torch.bfloat16, 2.0),
]


@pytest.mark.parametrize("case", CF_SMALL, ids=[c[0] for c in CF_SMALL])
def test_coarse_fine_full_parity(case):
    name, B, L, Hq, Hkv, D, C, tr, tg, dtype, a = case
    log(f"[coarse-fine] {name}")
    q, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, dtype, seed=400, qk_scale=a)
    o, lse = dca.coarse_fine_prefill(q.to(dev()), k.to(dev()), v.to(dev()), C, tr, tg, 1e4, return_lse=True)
    O, LSE = oracle.coarse_fine_prefill_ref(q, k, v, C, tr, tg, 1e4)
    mx, mean = assert_close(to_np(o), O, dtype, name)
    lerr = np.abs(to_np(lse) - LSE)
    assert np.all(lerr <= lse_bound_prefill(q, k, dtype)), (name, lerr.max())
    log(f"  O max {mx:.2e} mean {mean:.2e}  LSE max {lerr.max():.2e}")


CF_GPU_PLANTED = {   # (C, train, target, i, j*): fp32 any chunk, bf16 chunk % 64 == 0
    "f32_succ_frac": (12, 3, 7, 41, 30, torch.float32),
    "f32_inter_frac": (12, 3, 7, 60, 5, torch.float32),
    "bf16_intra": (64, 1, 8, 150, 140, torch.bfloat16),
    "bf16_succ": (64, 1, 8, 150, 100, torch.bfloat16),
    "bf16_inter": (64, 2, 5, 300, 17, torch.bfloat16),
}


@pytest.mark.parametrize("case", sorted(CF_GPU_PLANTED))
def test_coarse_fine_planted_keys(case):
    C, tr, tg, i, jstar, dtype = CF_GPU_PLANTED[case]
    D = 64
    q, k, v, want = cf_planted_case(C, tr, tg, i, jstar, D=D, seed=5)
    L = i + 70
    pad = lambda x: np.concatenate([x, np.random.default_rng(1).standard_normal((1, 70, 1, D)) * 0.1], 1)
    qt, kt, vt = (torch.from_numpy(pad(x)).to(dtype) for x in (q, k, v))
    o = to_np(dca.coarse_fine_prefill(qt.to(dev()), kt.to(dev()), vt.to(dev()), C, tr, tg, 1e4))
    O, _ = oracle.coarse_fine_prefill_ref(qt, kt, vt, C, tr, tg, 1e4, rows=[i])
    assert_close(o[:, i], O[:, 0], dtype, case)
    if dtype == torch.float32:
        assert np.abs(o[0, i, 0] - want).max() <= F32_TOL


def test_bf16_chunk_not_a_tile_multiple_is_rejected():
    q, k, v = (x.to(dev()) for x in inputs.prefill_inputs(1, 100, 1, 1, 64, "bf16", seed=1))
    with pytest.raises(dca.DCAError) as e:
        dca.coarse_fine_prefill(q, k, v, 48, 1, 4)
    assert e.value.status == dca._lib.DCA_ERR_UNSUPPORTED


def test_coarse_fine_32k_workload_sampled_rows():
    # The guide's parameters (C 512, 4096 -> 32768) on the 70B-shape 32k input.
    P = inputs.WORKLOADS["llama2_70b_32k"]
    B, L, Hq, Hkv, D = (P[x] for x in ("B", "L", "Hq", "Hkv", "D"))
    q, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, "bf16", seed=P["seed"])
    o = dca.coarse_fine_prefill(q.to(dev()), k.to(dev()), v.to(dev()), 512, 4096, 32768, P["base"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = sorted({0, 511, 512, 513, 1023, 1024, 1535, 16383, L - 1} | set(rng.integers(0, L, 8).tolist()))
    heads = [0, 13, 63]
    O, _ = oracle.coarse_fine_prefill_ref(q, k, v, 512, 4096, 32768, P["base"], rows=rows, heads=heads)
    mx, mean = assert_close(to_np(o[:, rows][:, :, heads]), O, torch.bfloat16, "coarse-fine 32k")
    log(f"  coarse_fine 32k O: max abs {mx:.3e}, mean abs {mean:.3e}")
