"""GPU parity of chunked prefill over a KV prefix and of ragged decode (through
the C ABI) against the fp64 oracle.

Definition: a chunk's new token r of sequence b is row pos0[b] + r of the DCA
prefill ("Dual-Chunk Attention: Training-Free 100k+ Context Guide", chunk
relations from absolute positions); a ragged decode is row kv_len[b] - 1 of
sequence b.  Cache rows past each sequence's valid length are filled with NaN,
so any read of them would show.  Bars: fp32 max-abs <= 1e-4; bf16 max-abs
<= 2e-2 and mean-abs <= 2e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs
from test_gpu_parity import assert_close, dev, log, lse_bound_prefill, to_np

pytestmark = pytest.mark.gpu


def make_caches(k, v, valid, c, w):
    """Rotated key cache (at j mod s) and value cache on the GPU, rows past
    valid[b] overwritten with NaN."""
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    vc = v.to(dev()).clone()
    for b, n in enumerate(valid):
        kc[b, n:] = float("nan")
        vc[b, n:] = float("nan")
    return kc, vc


CHUNK = [
    # name, B, Lq, pos0, q_len, cache_len, Hq, Hkv, D, c, w, dtype
    ("bf16_uniform_aligned", 2, 200, [256, 256], None, 600, 4, 2, 128, 256, 64, torch.bfloat16),
    ("bf16_unaligned_offsets", 2, 150, [100, 37], [150, 90], 300, 2, 1, 64, 128, 0, torch.bfloat16),
    ("bf16_ragged_aligned", 3, 300, [0, 64, 320], [300, 17, 129], 700, 8, 2, 128, 512, 128, torch.bfloat16),
    ("bf16_straddle_s96", 2, 100, [200, 50], [100, 60], 400, 2, 2, 128, 128, 32, torch.bfloat16),
    ("bf16_one_row", 2, 1, [499, 77], None, 500, 4, 1, 128, 256, 64, torch.bfloat16),
    ("bf16_70_sequences", 70, 8, [(b * 7) % 40 for b in range(70)], [b % 8 + 1 for b in range(70)],
     64, 2, 1, 64, 32, 8, torch.bfloat16),
    ("f32_ragged", 2, 70, [30, 100], [70, 20], 200, 2, 1, 64, 64, 16, torch.float32),
    ("f32_aligned_d128", 1, 96, [64], None, 200, 2, 2, 128, 128, 64, torch.float32),
]


@pytest.mark.parametrize("case", CHUNK, ids=[c[0] for c in CHUNK])
def test_prefill_chunk_matches_oracle(case):
    name, B, Lq, pos0, q_len, cache_len, Hq, Hkv, D, c, w, dtype = case
    log(f"[chunk] {name}")
    ql = [Lq] * B if q_len is None else q_len
    valid = [p + n for p, n in zip(pos0, ql)]
    qf, k, v = inputs.prefill_inputs(B, cache_len, Hq, Hkv, D, dtype, seed=300, qk_scale=2.0)
    q = torch.zeros(B, Lq, Hq, D, dtype=dtype)
    for b in range(B):
        q[b, : ql[b]] = qf[b, pos0[b]: pos0[b] + ql[b]]
    kc, vc = make_caches(k, v, valid, c, w)
    o, lse = dca.prefill_chunk(q.to(dev()), kc, vc, pos0, c, w, 1e4, q_len=q_len, return_lse=True)
    O, LSE = oracle.dca_prefill_chunk_ref(q, k, v, pos0, c, w, 1e4, q_len=ql)
    got, lg = to_np(o), to_np(lse)
    bound = lse_bound_prefill(qf, k, dtype)
    for b in range(B):
        n = ql[b]
        assert_close(got[b, :n], O[b, :n], dtype, f"{name} seq {b}")
        lb = bound if np.isscalar(bound) else bound[b][:, pos0[b]: pos0[b] + n]
        assert np.all(np.abs(lg[b, :, :n] - LSE[b, :, :n]) <= lb), (name, b)
        assert np.all(got[b, n:] == 0) and np.all(np.isneginf(lg[b, :, n:]))   # rows past q_len untouched


def test_chunks_concatenate_to_the_whole_prefill():
    B, L, Hq, Hkv, D, c, w = 1, 1000, 4, 2, 128, 256, 64
    q, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, "bf16", seed=301, qk_scale=2.0)
    whole = to_np(dca.prefill(q.to(dev()), k.to(dev()), v.to(dev()), c, w))
    kc, vc = make_caches(k, v, [L], c, w)
    parts = []
    for a, b in ((0, 300), (300, 301), (301, 600), (600, 1000)):   # aligned and unaligned offsets
        parts.append(to_np(dca.prefill_chunk(q[:, a:b].contiguous().to(dev()), kc, vc, a, c, w)))
    chunked = np.concatenate(parts, axis=1)
    O, _ = oracle.dca_prefill_ref(q, k, v, c, w)
    assert_close(chunked, O, torch.bfloat16, "chunked")
    assert np.abs(chunked - whole).max() <= 2e-2


DECODE_VAR = [
    # name, kv_len list, cache_len, Hq, Hkv, D, c, w, dtype
    ("bf16_ragged", [1, 77, 500, 1000, 333], 1000, 16, 2, 128, 512, 128, torch.bfloat16),
    ("bf16_d64_straddle", [257, 96, 95, 400], 400, 8, 8, 64, 128, 32, torch.bfloat16),
    ("f32_ragged", [50, 300, 7], 300, 4, 2, 64, 64, 16, torch.float32),
]


@pytest.mark.parametrize("case", DECODE_VAR, ids=[c[0] for c in DECODE_VAR])
def test_decode_varlen_matches_oracle(case):
    name, kv, cache_len, Hq, Hkv, D, c, w, dtype = case
    log(f"[decode varlen] {name}")
    B = len(kv)
    qd, k, v = inputs.decode_inputs(B, cache_len, Hq, Hkv, D, dtype, seed=302, qk_scale=2.0)
    kc, vc = make_caches(k, v, kv, c, w)
    o, lse = dca.decode_varlen(qd.to(dev()), kc, vc, kv, c, w, 1e4, return_lse=True)
    got = to_np(o)
    for b in range(B):
        Od, Ld = oracle.dca_decode_ref(qd[b: b + 1], k[b: b + 1, : kv[b]], v[b: b + 1, : kv[b]], c, w, 1e4)
        assert_close(got[b], Od[0], dtype, f"{name} seq {b}")
        # the uniform decode of that sequence alone gives the same row
        ou = dca.decode(qd[b: b + 1].to(dev()), kc[b: b + 1, : kv[b]].contiguous(),
                        vc[b: b + 1, : kv[b]].contiguous(), c, w, 1e4)
        assert np.abs(to_np(ou)[0] - got[b]).max() <= (1e-5 if dtype == torch.float32 else 2e-2)


def test_single_row_chunk_equals_ragged_decode():
    kv = [300, 1000, 45]
    B, cache_len, Hq, Hkv, D, c, w = 3, 1000, 8, 2, 128, 256, 64
    qd, k, v = inputs.decode_inputs(B, cache_len, Hq, Hkv, D, "bf16", seed=303, qk_scale=2.0)
    kc, vc = make_caches(k, v, kv, c, w)
    od = to_np(dca.decode_varlen(qd.to(dev()), kc, vc, kv, c, w))
    oc = to_np(dca.prefill_chunk(qd[:, None].contiguous().to(dev()), kc, vc, [n - 1 for n in kv], c, w))
    assert np.abs(oc[:, 0] - od).max() <= 2e-2


def test_chunked_prefill_32k_workload_last_chunk():
    # The 70B-shape 32k prompt prefilled as a final 4096-token chunk over a
    # 28672-token prefix.
    P = inputs.WORKLOADS["llama2_70b_32k"]
    B, L, Hq, Hkv, D, c, w = (P[x] for x in ("B", "L", "Hq", "Hkv", "D", "c", "w"))
    pos0 = L - 4096
    q, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, "bf16", seed=P["seed"])
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    o = dca.prefill_chunk(q[:, pos0:].contiguous().to(dev()), kc, v.to(dev()), pos0, c, w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = sorted({0, 1, 31, 32, 4095} | set(rng.integers(0, 4096, 10).tolist()))
    heads = [0, 9, 63]
    O, _ = oracle.dca_prefill_chunk_ref(q[:, pos0:], k, v, pos0, c, w, P["base"], rows=rows, heads=heads)
    mx, mean = assert_close(to_np(o[:, rows][:, :, heads]), O, torch.bfloat16, "chunk 32k")
    log(f"  chunked 32k last chunk O: max abs {mx:.3e}, mean abs {mean:.3e}")


def test_ragged_decode_100k_workload():
    P = inputs.WORKLOADS["decode_100k"]
    B, kvmax, Hq, Hkv, D, c, w = (P[x] for x in ("B", "kv_len", "Hq", "Hkv", "D", "c", "w"))
    kv = [int(x) for x in np.linspace(kvmax // 2, kvmax, B)]
    qd, k, v = inputs.decode_inputs(B, kvmax, Hq, Hkv, D, "bf16", seed=P["seed"])
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    o = to_np(dca.decode_varlen(qd.to(dev()), kc, v.to(dev()), kv, c, w))
    for b in (0, 7, 15):
        Od, _ = oracle.dca_decode_ref(qd[b: b + 1], k[b: b + 1, : kv[b]], v[b: b + 1, : kv[b]], c, w, P["base"])
        mx, mean = assert_close(o[b], Od[0], torch.bfloat16, f"ragged decode seq {b}")
        log(f"  ragged decode seq {b} (kv_len {kv[b]}): max abs {mx:.3e}")


def test_decode_more_sequences_than_one_launch_holds():
    # Ragged decodes launch in groups of 64 sequences (their lengths travel in
    # the kernel arguments): 70 sequences cross a group boundary.  Every row
    # must equal the uniform decode of that sequence alone; a few are checked
    # against the oracle too.  The same batch from page pools and under the
    # SelfExtend map gives the same bits as its dense form.
    B, cache_len, Hq, Hkv, D, c, w = 70, 300, 4, 2, 64, 128, 32
    kv = [1 + (b * 37) % cache_len for b in range(B)]
    qd, k, v = inputs.decode_inputs(B, cache_len, Hq, Hkv, D, "bf16", seed=304, qk_scale=2.0)
    kc, vc = make_caches(k, v, kv, c, w)
    o = dca.decode_varlen(qd.to(dev()), kc, vc, kv, c, w)
    for b in range(B):
        ou = dca.decode(qd[b: b + 1].to(dev()), kc[b: b + 1, : kv[b]].contiguous(),
                        vc[b: b + 1, : kv[b]].contiguous(), c, w)
        assert (ou[0].float() - o[b].float()).abs().max().item() <= 2e-2, b
    got = to_np(o)
    for b in (0, 63, 64, 69):
        Od, _ = oracle.dca_decode_ref(qd[b: b + 1], k[b: b + 1, : kv[b]], v[b: b + 1, : kv[b]], c, w, 1e4)
        assert_close(got[b], Od[0], torch.bfloat16, f"70 sequences, seq {b}")
    from test_gpu_paged import to_pages
    kp, table = to_pages(kc, kv, 16, seed=5)
    vp, _ = to_pages(vc, kv, 16, seed=5)
    assert torch.equal(dca.decode_paged(qd.to(dev()), kp, vp, table, kv, c, w), o)
    kg = k.to(dev())
    k_plain = dca.rope_remap(kg, dca.DCA_MAP_PLAIN, 1, 0)
    k_grp = dca.rope_remap(kg, dca.DCA_MAP_SE_KEY_GROUPED, 4, 50)
    se = dca.selfextend_decode(qd.to(dev()), k_plain, k_grp, vc, kv, 4, 50)
    O, _ = oracle.selfextend_decode_ref(qd, k, v, kv, 4, 50)
    sg = to_np(se)
    for b in (0, 63, 64, 69):
        assert_close(sg[b], O[b], torch.bfloat16, f"70 sequences selfextend, seq {b}")
