"""GPU parity of the paged-cache entry points (through the C ABI) against the
fp64 oracle, and against the dense entry points on the same rows.

A paged cache moves rows only: row j of sequence b is row j mod P of page
block_table[b][j // P] ("Dual-Chunk Attention: Training-Free 100k+ Context
Guide", "Strategic Recommendations": DCA in split-KV serving; the page layout
is the common block table).  Pages are handed out in a seeded random order
from a pool with spare pages; every pool row that no sequence may read is NaN,
so a stray read shows.  Bars: fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and
mean-abs <= 2e-3; against the dense entry points: bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs
from test_gpu_parity import assert_close, dev, log, to_np

pytestmark = pytest.mark.gpu


def to_pages(x, lengths, P, seed, spare=5):
    """Dense [B, L, H, D] -> (pool [num_pages, P, H, D], table int32 [B, nb]):
    sequence b's first lengths[b] rows in pages of P rows, pages shuffled;
    all other pool rows NaN."""
    B, L = x.shape[:2]
    nb = -(-max(lengths) // P)
    npages = B * nb + spare
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(npages)).long()
    pool = torch.full((npages, P) + tuple(x.shape[2:]), float("nan"), dtype=x.dtype, device=x.device)
    table = perm[: B * nb].view(B, nb).to(torch.int32)
    for b in range(B):
        for blk in range(-(-lengths[b] // P)):
            n = min(P, lengths[b] - blk * P)
            pool[int(table[b, blk])][:n] = x[b, blk * P: blk * P + n]
    return pool, table.to(x.device)


DECODE_PAGED = [
    # name, kv_len list, Hq, Hkv, D, c, w, page, dtype
    ("bf16_p16_ragged", [1, 77, 500, 1000, 333], 16, 2, 128, 512, 128, 16, torch.bfloat16),
    ("bf16_p64_gqa8", [4097, 3000, 129], 64, 8, 128, 1024, 256, 64, torch.bfloat16),
    ("bf16_p48_d64", [257, 96, 95, 400], 8, 8, 64, 128, 32, 48, torch.bfloat16),
    ("bf16_p256_one_page", [200, 256], 4, 1, 128, 256, 64, 256, torch.bfloat16),
    ("f32_p16", [50, 300, 7], 4, 2, 64, 64, 16, 16, torch.float32),
    ("f32_p32_d128", [100, 65], 2, 1, 128, 128, 32, 32, torch.float32),
]


@pytest.mark.parametrize("case", DECODE_PAGED, ids=[c[0] for c in DECODE_PAGED])
def test_decode_paged_matches_oracle_and_dense(case):
    name, kv, Hq, Hkv, D, c, w, P, dtype = case
    log(f"[decode paged] {name}")
    B, L = len(kv), max(kv)
    qd, k, v = inputs.decode_inputs(B, L, Hq, Hkv, D, dtype, seed=500, qk_scale=2.0)
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    vc = v.to(dev())
    kp, table = to_pages(kc, kv, P, seed=1)
    vp, _ = to_pages(vc, kv, P, seed=1)
    o, lse = dca.decode_paged(qd.to(dev()), kp, vp, table, kv, c, w, 1e4, return_lse=True)
    got = to_np(o)
    kraw, _ = to_pages(k, kv, P, seed=1)
    O, LSE = oracle.dca_decode_paged_ref(qd, to_np(kraw), to_np(to_pages(v, kv, P, seed=1)[0]), table.cpu().numpy(), kv,
                                         c, w, 1e4)
    for b in range(B):
        assert_close(got[b], O[b], dtype, f"{name} seq {b}")
    # the dense entry point on the same rows gives the same bits
    od, lsed = dca.decode_varlen(qd.to(dev()), kc, vc, kv, c, w, 1e4, return_lse=True)
    assert torch.equal(o, od) and torch.equal(lse, lsed)


CHUNK_PAGED = [
    # name, B, Lq, pos0, q_len, Hq, Hkv, D, c, w, page, dtype
    ("bf16_aligned_p64", 2, 200, [256, 512], None, 4, 2, 128, 256, 64, 64, torch.bfloat16),
    ("bf16_ragged_p16", 3, 150, [100, 37, 0], [150, 90, 1], 2, 1, 64, 128, 0, 16, torch.bfloat16),
    ("f32_p32", 2, 70, [30, 100], [70, 20], 2, 1, 64, 64, 16, 32, torch.float32),
]


@pytest.mark.parametrize("case", CHUNK_PAGED, ids=[c[0] for c in CHUNK_PAGED])
def test_prefill_chunk_paged_matches_oracle_and_dense(case):
    name, B, Lq, pos0, q_len, Hq, Hkv, D, c, w, P, dtype = case
    log(f"[chunk paged] {name}")
    ql = [Lq] * B if q_len is None else q_len
    valid = [p + n for p, n in zip(pos0, ql)]
    L = max(valid)
    qf, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, dtype, seed=501, qk_scale=2.0)
    q = torch.zeros(B, Lq, Hq, D, dtype=dtype)
    for b in range(B):
        q[b, : ql[b]] = qf[b, pos0[b]: pos0[b] + ql[b]]
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    vc = v.to(dev())
    kp, table = to_pages(kc, valid, P, seed=2)
    vp, _ = to_pages(vc, valid, P, seed=2)
    o, lse = dca.prefill_chunk_paged(q.to(dev()), kp, vp, table, pos0, c, w, 1e4, q_len=q_len, return_lse=True)
    O, _ = oracle.dca_prefill_chunk_paged_ref(q, to_np(to_pages(k, valid, P, seed=2)[0]),
                                              to_np(to_pages(v, valid, P, seed=2)[0]), table.cpu().numpy(), pos0, c, w,
                                              1e4, q_len=ql)
    got = to_np(o)
    for b in range(B):
        assert_close(got[b, : ql[b]], O[b, : ql[b]], dtype, f"{name} seq {b}")
    # dense caches with NaN past each sequence's rows: same bits
    kd, vd = kc.clone(), vc.clone()
    for b, n in enumerate(valid):
        kd[b, n:] = float("nan")
        vd[b, n:] = float("nan")
    od, lsed = dca.prefill_chunk(q.to(dev()), kd, vd, pos0, c, w, 1e4, q_len=q_len, return_lse=True)
    assert torch.equal(o, od) and torch.equal(lse, lsed)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_out_of_pool_table_entry_poisons_only_its_sequence(dtype):
    # An entry outside [0, num_pages) is never dereferenced: the sequence that
    # names it gets NaN, the others are unchanged.
    kv, Hq, Hkv, D, c, w, P = [300, 300, 300], 8, 2, 64, 128, 32, 16
    qd, k, v = inputs.decode_inputs(3, 300, Hq, Hkv, D, dtype, seed=502, qk_scale=2.0)
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    kp, table = to_pages(kc, kv, P, seed=3)
    vp, _ = to_pages(v.to(dev()), kv, P, seed=3)
    good = dca.decode_paged(qd.to(dev()), kp, vp, table, kv, c, w)
    bad_table = table.clone()
    bad_table[1, 5] = kp.shape[0] + 7
    bad = dca.decode_paged(qd.to(dev()), kp, vp, bad_table, kv, c, w)
    assert torch.isnan(bad[1]).all()
    assert torch.equal(bad[0], good[0]) and torch.equal(bad[2], good[2])
    bad_table[1, 5] = -1
    assert torch.isnan(dca.decode_paged(qd.to(dev()), kp, vp, bad_table, kv, c, w)[1]).all()


def test_decode_paged_100k_workload():
    # decode_100k's shape with ragged lengths in 64-row pages, sampled sequences
    P_ = inputs.WORKLOADS["decode_100k"]
    B, kvmax, Hq, Hkv, D, c, w = (P_[x] for x in ("B", "kv_len", "Hq", "Hkv", "D", "c", "w"))
    kv = [int(x) for x in np.linspace(kvmax // 2, kvmax, B)]
    qd, k, v = inputs.decode_inputs(B, kvmax, Hq, Hkv, D, "bf16", seed=P_["seed"])
    kc = dca.rope_remap(k.to(dev()), dca.DCA_MAP_KEY, c, w)
    kp, table = to_pages(kc, kv, 64, seed=4)
    del kc
    vp, _ = to_pages(v.to(dev()), kv, 64, seed=4)
    o = to_np(dca.decode_paged(qd.to(dev()), kp, vp, table, kv, c, w))
    for b in (0, 9, 15):
        Od, _ = oracle.dca_decode_ref(qd[b: b + 1], k[b: b + 1, : kv[b]], v[b: b + 1, : kv[b]], c, w, P_["base"])
        mx, _ = assert_close(o[b], Od[0], torch.bfloat16, f"paged decode seq {b}")
        log(f"  paged decode seq {b} (kv_len {kv[b]}): max abs {mx:.3e}")


MAP_PAGED = [
    # name, map, kv list, Hq, Hkv, D, params, page, dtype
    ("se_bf16_p16", "selfextend", [1, 50, 99, 100, 101, 700], 8, 2, 128, (4, 100), 16, torch.bfloat16),
    ("se_bf16_p48_long", "selfextend", [4097, 2500, 9000], 64, 8, 128, (8, 1024), 48, torch.bfloat16),
    ("se_f32_p32", "selfextend", [1, 34, 35, 600], 4, 2, 64, (5, 33), 32, torch.float32),
    ("cf_bf16_p16", "coarse_fine", [1, 64, 65, 128, 129, 700], 8, 2, 128, (64, 1, 8), 16, torch.bfloat16),
    ("cf_bf16_p64_guide", "coarse_fine", [600, 2048, 5000], 16, 2, 128, (512, 4096, 32768), 64, torch.bfloat16),
    ("cf_f32_p16", "coarse_fine", [1, 13, 14, 27, 400], 4, 2, 64, (13, 2, 9), 16, torch.float32),
]


@pytest.mark.parametrize("case", MAP_PAGED, ids=[c[0] for c in MAP_PAGED])
def test_map_decode_paged_matches_oracle_and_dense(case):
    # Both rotated key pools and the value pool share one block table (the same
    # page order for all three).  Oracle from the raw keys; the dense map decode
    # on the same rows gives the same bits.
    name, which, kv, Hq, Hkv, D, params, P, dtype = case
    log(f"[map decode paged] {name}")
    B, L = len(kv), max(kv)
    qd, k, v = inputs.decode_inputs(B, L, Hq, Hkv, D, dtype, seed=503, qk_scale=2.0)
    kg = k.to(dev())
    k_plain = dca.rope_remap(kg, dca.DCA_MAP_PLAIN, 1, 0)
    if which == "selfextend":
        G, W = params
        k_2nd = dca.rope_remap(kg, dca.DCA_MAP_SE_KEY_GROUPED, G, W)
        dense = lambda: dca.selfextend_decode(qd.to(dev()), k_plain, k_2nd, v.to(dev()), kv, G, W, return_lse=True)
        paged = lambda a, b_, c_, t: dca.selfextend_decode_paged(qd.to(dev()), a, b_, c_, t, kv, G, W,
                                                                  return_lse=True)
        O, _ = oracle.selfextend_decode_ref(qd, k, v, kv, G, W)
    else:
        C, tr, tg = params
        k_2nd = dca.coarse_fine_key_remap(kg, C, tr, tg)
        dense = lambda: dca.coarse_fine_decode(qd.to(dev()), k_plain, k_2nd, v.to(dev()), kv, C, tr, tg,
                                               return_lse=True)
        paged = lambda a, b_, c_, t: dca.coarse_fine_decode_paged(qd.to(dev()), a, b_, c_, t, kv, C, tr, tg,
                                                                   return_lse=True)
        O, _ = oracle.coarse_fine_decode_ref(qd, k, v, kv, C, tr, tg)
    kp, table = to_pages(k_plain, kv, P, seed=7)
    k2p, _ = to_pages(k_2nd, kv, P, seed=7)
    vp, _ = to_pages(v.to(dev()), kv, P, seed=7)
    o, lse = paged(kp, k2p, vp, table)
    got = to_np(o)
    for b in range(B):
        assert_close(got[b], O[b], dtype, f"{name} seq {b}")
    od, lsed = dense()
    assert torch.equal(o, od) and torch.equal(lse, lsed)
    # an entry outside the pool poisons only its own sequence
    bad_table = table.clone()
    bad_table[B - 1, 0] = kp.shape[0] + 3
    ob, _ = paged(kp, k2p, vp, bad_table)
    assert torch.isnan(ob[B - 1]).all()
    assert torch.equal(ob[: B - 1], o[: B - 1])
