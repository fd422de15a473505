"""dca_decode_paged_noalloc (the entry point that allocates nothing) against
dca_decode_paged, through the C ABI, on two calls in a row (the second with
a smaller input, so it runs on scratch the first call left behind), and
against the fp64 oracle at the bf16 / fp32 bars (max-abs 2e-2, mean-abs
2e-3; fp32 1e-4).  The two entry points share their kernels, so their outputs
must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs
from test_gpu_paged import to_pages
from test_gpu_parity import assert_close, dev, log, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # name, kv_len list, Hq, Hkv, D, c, w, page, dtype
    ("bf16_gqa8_ragged", [4097, 3000, 129, 1, 2500], 64, 8, 128, 1024, 256, 16, torch.bfloat16),
    ("bf16_smaller", [300, 57], 16, 2, 64, 128, 32, 32, torch.bfloat16),
    ("f32_smallest", [40, 17], 4, 2, 64, 64, 16, 16, torch.float32),
]


def run_case(case, seed):
    name, kv, Hq, Hkv, D, c, w, P, dtype = case
    log(f"[decode paged noalloc] {name}")
    B, L = len(kv), max(kv)
    qd, k, v = inputs.decode_inputs(B, L, Hq, Hkv, D, dtype, seed=seed, qk_scale=2.0)
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    kp, table = to_pages(kc, kv, P, seed=seed)
    vp, _ = to_pages(v.to(dev()), kv, P, seed=seed)
    q = qd.to(dev())
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev())
    got, got_lse = dca.decode_paged_noalloc(q, kp, vp, table, kv, c, w, 1e4, out=out, lse=lse)
    assert got is out and got_lse is lse
    want, want_lse = dca.decode_paged(q, kp, vp, table, kv, c, w, 1e4, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(got, want) and torch.equal(got_lse, want_lse), name
    kraw, _ = to_pages(k, kv, P, seed=seed)
    O, _ = oracle.dca_decode_paged_ref(qd, to_np(kraw), to_np(to_pages(v, kv, P, seed=seed)[0]),
                                       table.cpu().numpy(), kv, c, w, 1e4)
    g = to_np(got)
    for b in range(B):
        assert_close(g[b], O[b], dtype, f"{name} seq {b}")


def test_noalloc_matches_workspace_decode_two_calls():
    # largest first, then smaller: the later calls reuse the scratch the first left
    for i, case in enumerate(CASES):
        run_case(case, seed=900 + i)


def test_noalloc_refuses_oversized_call_before_launch():
    # 64 sequences x 1024 query heads need more than the static scratch; refused
    # on the host with DCA_ERR_TOO_LARGE, nothing enqueued
    B, Hq, Hkv, D, P = 64, 1024, 8, 128, 16
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device=dev())
    pool = torch.zeros(B, P, Hkv, D, dtype=torch.bfloat16, device=dev())
    table = torch.arange(B, dtype=torch.int32, device=dev()).view(B, 1)
    with pytest.raises(dca.DCAError) as e:
        dca.decode_paged_noalloc(q, pool, pool, table, [P] * B, 4096, 1024)
    assert e.value.status == -5
