"""Pins of the coarse / fine map oracle (the DCA guide's own formulas).

Source: "Dual-Chunk Attention: Training-Free 100k+ Context Guide", sections
"Inter-Chunk Attention" and "Successive Chunk Smoothing", and the pairs its
"End-to-End Implementation" script inspects (C = 512, L_train = 4096,
L_target = 32768, kappa = 8).  Expected values below are worked out by hand
from those formulas (the page prints the pairs but not the numbers), or are
properties the page states: intra pairs unscaled, the successive ramp
beginning at the plain distance at the chunk edge, the fine offset keeping
order inside the key's chunk, and no distance above L_train over a 16k
horizon.
"""
import math

import numpy as np
import pytest

import oracle.coarse_fine_ref as cf
from long_context_attention_dca_amd import inputs
from test_oracle_pins import _rope_complex, _sdpa_plain_rope

GUIDE = dict(C=512, train_len=4096, target_len=32768)


def _table_entry(i, j, C=512, train_len=4096, target_len=32768):
    return cf.coarse_fine_distance_table(i + 1, C, train_len, target_len)[i, j]


def test_guide_pairs_by_hand():
    # (100, 98): same chunk -> i - j = 2.  (511, 0): same chunk -> 511.
    assert _table_entry(100, 98) == 2.0
    assert _table_entry(511, 0) == 511.0
    # (600, 400): adjacent chunks; lambda = 88/512 = 0.171875; inter value
    # 1 * 512/8 + (88 - 400) = -248; (1 - 0.171875) * 200 + 0.171875 * (-248)
    # = 165.625 - 42.625 = 123.
    assert _table_entry(600, 400) == pytest.approx(123.0, abs=1e-12)


def test_guide_far_pair_and_bound_by_hand():
    # (16383, 0): chunks 31 and 0 -> 31 * 64 + 511 = 2495 (form A positions,
    # checked against form B on a smaller horizon below).
    _, _, p_inter = cf.coarse_fine_positions(16383, **GUIDE)
    _, k_sc = cf.coarse_fine_key_positions(0, **GUIDE)
    assert p_inter - k_sc == 2495.0
    # The page's invariant over its 16k horizon: no distance above L_train.
    # Per row the largest distance is at the smallest key position of each
    # relation's key range: o_i (intra), P_succ - (c_i - 1) C (successive),
    # P_inter - 0 (inter).
    i = np.arange(16384)
    c, o = i // 512, i % 512
    p_intra, p_succ, p_inter = cf.coarse_fine_positions(i, **GUIDE)
    row_max = np.maximum.reduce([o.astype(float), np.where(c >= 1, p_succ - (c - 1) * 512, -np.inf),
                                 np.where(c >= 2, p_inter, -np.inf)])
    assert row_max.max() == 2495.0 and row_max.max() <= 4096
    # ... which the same map breaks at the target length: row 32767 reaches
    # 63 * 64 + 511 = 4543 > 4096, and (1024, 511) gives 2 * 64 - 511 = -383.
    _, _, p_last = cf.coarse_fine_positions(32767, **GUIDE)
    assert p_last == 4543.0
    assert _table_entry(1024, 511) == -383.0


@pytest.mark.parametrize("C,train,target,L", [(16, 4, 8, 90), (12, 3, 7, 70), (8, 2, 2, 40), (5, 1, 3, 33)])
def test_factorized_positions_equal_the_guide_formulas(C, train, target, L):
    M = cf.coarse_fine_distance_table(L, C, train, target)
    ii, jj = np.tril_indices(L)
    pq = np.stack(cf.coarse_fine_positions(ii, C, train, target))
    kp_plain, kp_scaled = cf.coarse_fine_key_positions(jj, C, train, target)
    rho = ii // C - jj // C
    cls = np.minimum(rho, 2)
    got = pq[cls, np.arange(len(ii))] - np.where(cls == 2, kp_scaled, kp_plain)
    assert np.abs(got - M[ii, jj]).max() < 1e-9


def test_page_stated_properties():
    C, train, target, L = 16, 4, 12, 120
    M = cf.coarse_fine_distance_table(L, C, train, target)
    for i in range(L):
        for j in range(i + 1):
            if i // C == j // C:
                assert M[i, j] == i - j                        # intra: unscaled
            if i // C == j // C + 1 and i % C == 0:
                assert M[i, j] == i - j                        # ramp starts from the local distance
            if i // C >= j // C + 2 and j % C < C - 1 and j + 1 <= i:
                assert M[i, j] - M[i, j + 1] == pytest.approx(1.0)   # fine offset keeps order in the chunk


@pytest.mark.parametrize("C,L,Hq,Hkv,D", [(16, 80, 2, 1, 32), (7, 50, 2, 2, 16)])
def test_kappa_one_is_plain_rope(C, L, Hq, Hkv, D):
    q, k, v = inputs.prefill_inputs(1, L, Hq, Hkv, D, "f32", seed=41, qk_scale=2.0)
    O, _ = cf.coarse_fine_prefill_ref(q, k, v, C, 100, 100)
    want = _sdpa_plain_rope(q, k, v, 10000.0, 1 / math.sqrt(D))
    assert np.abs(O - want).max() < 1e-12


@pytest.mark.parametrize("C,train,target,L,Hq,Hkv,D", [(16, 4, 8, 70, 2, 1, 16), (12, 3, 7, 50, 1, 1, 8),
                                                       (10, 1, 4, 45, 2, 2, 8)])
def test_formA_equals_formB(C, train, target, L, Hq, Hkv, D):
    q, k, v = inputs.prefill_inputs(1, L, Hq, Hkv, D, "f32", seed=42, qk_scale=2.0)
    OA, LA = cf.coarse_fine_prefill_ref(q, k, v, C, train, target)
    OB, LB = cf.coarse_fine_prefill_formB(q, k, v, C, train, target)
    assert np.abs(OA - OB).max() < 1e-12 and np.abs(LA - LB).max() < 1e-12


def cf_planted_case(C, train, target, i, jstar, D=16, seed=0, target_logit=3.0):
    """k_{j*} = alpha R_{M*} q_i with M* the worked-out distance: logit of j* is
    target_logit, the others 0; O_i in closed form."""
    rng = np.random.default_rng(seed)
    L = i + 1
    q = rng.standard_normal((1, L, 1, D))
    v = rng.standard_normal((1, L, 1, D))
    k = np.zeros((1, L, 1, D))
    Mstar = _table_entry(i, jstar, C, train, target)
    alpha = target_logit / ((1 / math.sqrt(D)) * float(q[0, i, 0] @ q[0, i, 0]))
    k[0, jstar, 0] = alpha * _rope_complex(q[0, i, 0], Mstar, 1e4)
    e = math.exp(target_logit)
    want = (e * v[0, jstar, 0] + v[0, :L, 0].sum(0) - v[0, jstar, 0]) / (e + i)
    return q, k, v, want


CF_PLANTED = {
    "intra": (16, 4, 8, 40, 35),
    "succ": (16, 4, 8, 40, 20),
    "succ_frac": (12, 3, 7, 41, 30),
    "inter": (16, 4, 8, 70, 9),
    "inter_frac": (12, 3, 7, 60, 5),
}


@pytest.mark.parametrize("case", sorted(CF_PLANTED))
def test_planted_key_closed_form(case):
    C, train, target, i, jstar = CF_PLANTED[case]
    q, k, v, want = cf_planted_case(C, train, target, i, jstar)
    O, _ = cf.coarse_fine_prefill_ref(q, k, v, C, train, target, rows=[i])
    assert np.abs(O[0, 0, 0] - want).max() < 1e-12


def test_pins_catch_a_ramp_weight_from_the_key(monkeypatch):
    def wrong(L, C, train, target):   # lambda from the key's offset instead of the query's
        kappa = target / train
        M = np.full((L, L), np.nan)
        for i in range(L):
            for j in range(i + 1):
                ci, oi = divmod(i, C)
                cj, oj = divmod(j, C)
                inter = (ci - cj) * C / kappa + (oi - oj)
                lam = oj / C
                M[i, j] = i - j if ci == cj else ((1 - lam) * (i - j) + lam * inter if ci == cj + 1 else inter)
        return M
    monkeypatch.setattr(cf, "coarse_fine_distance_table", wrong)
    with pytest.raises(AssertionError):
        test_guide_pairs_by_hand()


def test_pins_catch_a_scaled_fine_offset(monkeypatch):
    orig = cf.coarse_fine_positions

    def wrong(i, C, train_len, target_len):   # scaling the whole position (PI-like) for inter pairs
        a, b, _ = orig(i, C, train_len, target_len)
        return a, b, np.asarray(i, dtype=float) * train_len / target_len
    monkeypatch.setattr(cf, "coarse_fine_positions", wrong)
    with pytest.raises(AssertionError):
        test_guide_far_pair_and_bound_by_hand()


@pytest.mark.parametrize("C,train,target", [(16, 4, 8), (12, 3, 7), (8, 2, 2)])
def test_decode_is_the_last_prefill_row(C, train, target):
    kv = [1, 20, 61, 50]
    B, L, Hq, Hkv, D = len(kv), max(kv), 4, 2, 16
    q, k, v = (x.double().numpy() for x in inputs.prefill_inputs(B, L, Hq, Hkv, D, "f32", seed=62, qk_scale=2.0))
    qd = np.stack([q[b, kv[b] - 1] for b in range(B)])
    O, LSE = cf.coarse_fine_decode_ref(qd, k, v, kv, C, train, target)
    for b in range(B):
        n = kv[b]
        Op, Lp = cf.coarse_fine_prefill_ref(q[b: b + 1, :n], k[b: b + 1, :n], v[b: b + 1, :n], C, train, target,
                                            rows=[n - 1])
        assert np.abs(O[b] - Op[0, 0]).max() < 1e-12 and np.abs(LSE[b] - Lp[0, :, 0]).max() < 1e-12


def test_scaled_key_remap_gives_the_guide_distances():
    # For a pair two or more chunks apart, the inter query position against the
    # remapped key reproduces the guide's distance: <R_{P_inter(i)} q, remap(k)_j>
    # = q . R_{-M(i, j)} k with M from the per-pair formulas.
    C, train, target, L, D = 10, 3, 8, 47, 8
    rng = np.random.default_rng(63)
    q = rng.standard_normal(D)
    k = rng.standard_normal((1, L, 1, D))
    kr = cf.coarse_fine_key_remap_ref(k, 0, C, train, target)[0, :, 0]
    M = cf.coarse_fine_distance_table(L, C, train, target)
    i = L - 1
    _, _, p_inter = cf.coarse_fine_positions(i, C, train, target)
    qr = _rope_complex(q, p_inter, 1e4)
    for j in range(0, (i // C - 1) * C):
        want = float(q @ _rope_complex(k[0, j, 0], -M[i, j], 1e4))
        assert abs(float(qr @ kr[j]) - want) < 1e-9, j
    # pos0 shifts the positions: rows of a later slice match the whole remap
    whole = cf.coarse_fine_key_remap_ref(k, 0, C, train, target)
    assert np.abs(cf.coarse_fine_key_remap_ref(k[:, 13:], 13, C, train, target) - whole[:, 13:]).max() < 1e-12
