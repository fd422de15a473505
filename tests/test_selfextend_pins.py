"""Pins of the SelfExtend (grouped / neighbor) oracle against facts outside it.

Source: "LLM Maybe LongLM: Self-Extend LLM Context Window Without Tuning"
(abstract): grouped attention for far-apart tokens, neighbor attention within a
chosen range.  What fixes each expected value: plain RoPE attention through
PyTorch's fp64 SDPA (group size 1, or a window covering the sequence, where the
two levels coincide with ordinary attention), the brute-force position table,
invariants of the grouped map, and a planted key with a closed-form output.
A final group plants plausible mistakes in the oracle and checks the pins
catch them.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.selfextend_ref as se
from long_context_attention_dca_amd import inputs
from test_oracle_pins import _rope_complex, _sdpa_plain_rope


# ------------------------------------------------------ reduces to plain RoPE -
@pytest.mark.parametrize("W,L,Hq,Hkv,D", [(0, 60, 2, 1, 32), (5, 77, 2, 2, 16), (40, 50, 4, 2, 16)])
def test_group_size_one_is_plain_rope(W, L, Hq, Hkv, D):
    # G = 1: grouped positions are i + W - W = i and j, i.e. ordinary RoPE.
    q, k, v = inputs.prefill_inputs(1, L, Hq, Hkv, D, "f32", seed=21, qk_scale=2.0)
    O, _ = oracle.selfextend_prefill_ref(q, k, v, 1, W)
    want = _sdpa_plain_rope(q, k, v, 10000.0, 1 / math.sqrt(D))
    assert np.abs(O - want).max() < 1e-12


@pytest.mark.parametrize("G,L", [(4, 64), (7, 90)])
def test_window_covering_the_sequence_is_plain_rope(G, L):
    q, k, v = inputs.prefill_inputs(1, L, 2, 1, 16, "f32", seed=22, qk_scale=2.0)
    O, _ = oracle.selfextend_prefill_ref(q, k, v, G, L)
    want = _sdpa_plain_rope(q, k, v, 10000.0, 1 / math.sqrt(16))
    assert np.abs(O - want).max() < 1e-12


def test_rows_inside_the_window_are_plain_and_later_rows_are_not():
    G, W, L, D = 4, 24, 120, 16
    q, k, v = inputs.prefill_inputs(1, L, 1, 1, D, "f32", seed=23, qk_scale=2.0)
    plain = _sdpa_plain_rope(q, k, v, 10000.0, 1 / math.sqrt(D))
    O, _ = oracle.selfextend_prefill_ref(q, k, v, G, W, rows=np.arange(W))
    assert np.abs(O - plain[:, :W]).max() < 1e-12
    O2, _ = oracle.selfextend_prefill_ref(q, k, v, G, W, rows=[L - 1])
    assert np.abs(O2[:, 0] - plain[:, L - 1]).max() > 1e-3


# ---------------------------------------------------------------- two forms -
@pytest.mark.parametrize("G,W,L,Hq,Hkv,D", [(3, 7, 40, 2, 1, 16), (4, 0, 33, 1, 1, 8),
                                            (2, 9, 50, 2, 2, 8), (8, 16, 70, 1, 1, 16)])
def test_formA_equals_formB(G, W, L, Hq, Hkv, D):
    q, k, v = inputs.prefill_inputs(1, L, Hq, Hkv, D, "f32", seed=24, qk_scale=2.0)
    OA, LA = oracle.selfextend_prefill_ref(q, k, v, G, W)
    OB, LB = oracle.selfextend_prefill_formB(q, k, v, G, W)
    assert np.abs(OA - OB).max() < 1e-12
    assert np.abs(LA - LB).max() < 1e-12


# ------------------------------------------------------------ position table -
@pytest.mark.parametrize("G,W,L", [(4, 10, 80), (3, 3, 50), (8, 0, 40), (1, 6, 30), (5, 12, 64)])
def test_position_table_properties(G, W, L):
    M = se.se_relative_position_table(L, G, W)
    for i in range(L):
        for j in range(i + 1):
            if i - j < W:
                assert M[i, j] == i - j                       # neighbors: exact distance
            else:
                assert M[i, j] >= W                           # grouped: never inside the window
                assert M[i, j] == M[i, (j // G) * G]          # depends on j only via floor(j/G)
                assert M[i, j] <= (i - j) // G + W - W // G + 1
    # the vectorised helpers give the same table
    ii, jj = np.tril_indices(L)
    rel = se.se_relation(ii, jj, W)
    Mv = se.se_query_position(ii, G, W, rel) - se.se_key_position(jj, G, rel)
    assert np.array_equal(Mv, M[ii, jj])


def test_grouped_distance_continues_the_window_edge():
    # i, j multiples of G at distance exactly W: the grouped distance is W.
    for G, W in ((4, 16), (8, 64), (3, 9)):
        for j in (0, G, 5 * G):
            i = j + W
            assert se.se_relative_position_table(i + 1, G, W)[i, j] == W


def test_remap_positions():
    t = np.arange(12)
    assert list(se.se_remap_positions(t, se.MAP_SE_KEY_GROUPED, 4, 6)) == [0] * 4 + [1] * 4 + [2] * 4
    assert list(se.se_remap_positions(t, se.MAP_SE_Q_GROUPED, 4, 6)) == [5] * 4 + [6] * 4 + [7] * 4


# ------------------------------------------------------------ group invariance
def test_swapping_two_keys_of_one_group_leaves_the_row_unchanged():
    G, W, L, D = 4, 16, 90, 16
    q, k, v = inputs.prefill_inputs(1, L, 1, 1, D, "f32", seed=25, qk_scale=2.0)
    i, j1, j2 = 89, 40, 43                      # floor(40/4) == floor(43/4); both <= i - W
    k2, v2 = k.clone(), v.clone()
    k2[:, [j1, j2]] = k[:, [j2, j1]]
    v2[:, [j1, j2]] = v[:, [j2, j1]]
    O, _ = oracle.selfextend_prefill_ref(q, k, v, G, W, rows=[i])
    Os, _ = oracle.selfextend_prefill_ref(q, k2, v2, G, W, rows=[i])
    assert np.abs(O - Os).max() < 1e-12
    # ... not so under plain RoPE, nor for keys of different groups
    plain = _sdpa_plain_rope(q, k, v, 10000.0, 1 / math.sqrt(D))[:, i]
    plain_s = _sdpa_plain_rope(q, k2, v2, 10000.0, 1 / math.sqrt(D))[:, i]
    assert np.abs(plain - plain_s).max() > 1e-4
    k3, v3 = k.clone(), v.clone()
    k3[:, [j1, 44]] = k[:, [44, j1]]
    v3[:, [j1, 44]] = v[:, [44, j1]]
    O3, _ = oracle.selfextend_prefill_ref(q, k3, v3, G, W, rows=[i])
    assert np.abs(O - O3).max() > 1e-4


# ------------------------------------------------------------- planted keys -
def se_planted_case(G, W, i, jstar, D=16, seed=0, target_logit=3.0):
    """All keys zero except k_{j*} = alpha R_{M*} q_i, with M* the distance the
    relation of (i, j*) gives: the logit of j* is target_logit, every other
    logit 0, and O_i = (e^T v_{j*} + sum_{j != j*} v_j) / (e^T + i)."""
    rng = np.random.default_rng(seed)
    L = i + 1
    q = rng.standard_normal((1, L, 1, D))
    v = rng.standard_normal((1, L, 1, D))
    k = np.zeros((1, L, 1, D))
    if i - jstar < W:
        Mstar = i - jstar
    else:
        Mstar = (i // G + W - W // G) - jstar // G
    alpha = target_logit / ((1 / math.sqrt(D)) * float(q[0, i, 0] @ q[0, i, 0]))
    k[0, jstar, 0] = alpha * _rope_complex(q[0, i, 0], Mstar, 1e4)
    e = math.exp(target_logit)
    want = (e * v[0, jstar, 0] + v[0, :L, 0].sum(0) - v[0, jstar, 0]) / (e + i)
    return q, k, v, want


SE_PLANTED = {
    "neighbor": (4, 16, 60, 50),
    "neighbor_edge": (4, 16, 60, 45),       # i - j = W - 1
    "grouped_edge": (4, 16, 60, 44),        # i - j = W (W a multiple of G: M = W, continuous)
    "grouped_edge_unaligned": (4, 14, 64, 50),  # i - j = W, M = 15 != W: catches an edge off by one
    "grouped_far": (4, 16, 97, 13),
    "grouped_g7": (7, 10, 80, 22),
}


@pytest.mark.parametrize("case", sorted(SE_PLANTED))
def test_planted_key_closed_form(case):
    G, W, i, jstar = SE_PLANTED[case]
    q, k, v, want = se_planted_case(G, W, i, jstar)
    O, _ = oracle.selfextend_prefill_ref(q, k, v, G, W, rows=[i])
    assert np.abs(O[0, 0, 0] - want).max() < 1e-12


# ---------------------------------------------------------- planted mistakes -
def _caught():
    for case, (G, W, i, jstar) in SE_PLANTED.items():
        q, k, v, want = se_planted_case(G, W, i, jstar)
        O, _ = oracle.selfextend_prefill_ref(q, k, v, G, W, rows=[i])
        if np.abs(O[0, 0, 0] - want).max() > 1e-6:
            return True
    return False


def test_pins_catch_a_missing_query_shift(monkeypatch):
    monkeypatch.setattr(se, "se_query_position",
                        lambda i, G, W, rel: np.where(np.asarray(rel) == se.GROUPED,
                                                      np.asarray(i) // G, np.asarray(i)))
    assert _caught()


def test_pins_catch_an_off_by_one_window(monkeypatch):
    monkeypatch.setattr(se, "se_relation",
                        lambda i, j, W: np.where(np.asarray(i) - np.asarray(j) <= W, se.NEIGHBOR,
                                                 se.GROUPED))
    assert _caught()


def test_pins_catch_ungrouped_keys(monkeypatch):
    monkeypatch.setattr(se, "se_key_position", lambda j, G, rel: np.asarray(j, dtype=np.int64))
    assert _caught()


@pytest.mark.parametrize("G,W", [(4, 16), (3, 0), (1, 7), (5, 200)])
def test_decode_is_the_last_prefill_row(G, W):
    # A ragged batch: sequence b decodes its token kv[b] - 1 over its first kv[b] keys.
    kv = [1, 37, 90, 64]
    B, L, Hq, Hkv, D = len(kv), max(kv), 4, 2, 16
    q, k, v = (x.double().numpy() for x in inputs.prefill_inputs(B, L, Hq, Hkv, D, "f32", seed=61, qk_scale=2.0))
    qd = np.stack([q[b, kv[b] - 1] for b in range(B)])
    O, LSE = oracle.selfextend_decode_ref(qd, k, v, kv, G, W)
    for b in range(B):
        n = kv[b]
        Op, Lp = oracle.selfextend_prefill_ref(q[b: b + 1, :n], k[b: b + 1, :n], v[b: b + 1, :n], G, W,
                                               rows=[n - 1])
        assert np.abs(O[b] - Op[0, 0]).max() < 1e-12 and np.abs(LSE[b] - Lp[0, :, 0]).max() < 1e-12
