"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a closed form, a library
routine (PyTorch's SDPA in fp64), an invariant the DCA guide states, a value
the DCA guide prints, or brute force on tiny inputs.  A final group plants
plausible mistakes in the oracle (on the CPU) and checks that the pins catch
them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.dca_ref as ref
from long_context_attention_dca_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- RoPE ------
def test_rope_closed_form_d2():
    # theta_0 = base^0 = 1 for any base: a pure planar rotation by p radians.
    for p in (0.0, 0.5, 3.0, -1.25):
        out = oracle.rope_rotate(np.array([1.0, 0.0]), p, 10000.0)
        assert np.allclose(out, [math.cos(p), math.sin(p)], atol=1e-15)
        out = oracle.rope_rotate(np.array([0.0, 1.0]), p, 500.0)
        assert np.allclose(out, [-math.sin(p), math.cos(p)], atol=1e-15)


def test_rope_closed_form_d4_pairing_and_frequencies():
    # D = 4, base = 100: theta = (1, 0.1); pairs are (x0, x2) and (x1, x3).
    x = np.array([1.0, 2.0, 3.0, 4.0])
    p = 2.0
    a0, a1 = p * 1.0, p * 0.1
    want = [1 * math.cos(a0) - 3 * math.sin(a0),
            2 * math.cos(a1) - 4 * math.sin(a1),
            3 * math.cos(a0) + 1 * math.sin(a0),
            4 * math.cos(a1) + 2 * math.sin(a1)]
    assert np.allclose(oracle.rope_rotate(x, p, 100.0), want, atol=1e-14)


def _rope_complex(x, pos, base):
    """Independent formulation: the rotary pair as one complex number."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    theta = np.exp(-np.log(base) * (2.0 * np.arange(half) / x.shape[-1]))
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * np.asarray(pos, float)[..., None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_matches_complex_form_and_relative_identity():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 64))
    y = rng.standard_normal((7, 64))
    pos = rng.integers(0, 5000, size=7)
    assert np.allclose(oracle.rope_rotate(x, pos, 1e4), _rope_complex(x, pos, 1e4), atol=1e-12)
    # Rotations preserve norms and compose additively.
    assert np.allclose(np.linalg.norm(oracle.rope_rotate(x, pos, 1e4), axis=-1),
                       np.linalg.norm(x, axis=-1), atol=1e-12)
    a, b = 37, 1234
    assert np.allclose(oracle.rope_rotate(oracle.rope_rotate(x, a, 1e4), b, 1e4),
                       oracle.rope_rotate(x, a + b, 1e4), atol=1e-11)
    # Score depends only on the relative position (the guide's RoPE identity).
    lhs = np.sum(oracle.rope_rotate(x, a, 1e4) * oracle.rope_rotate(y, b, 1e4), axis=-1)
    rhs = np.sum(x * oracle.rope_rotate(y, b - a, 1e4), axis=-1)
    assert np.allclose(lhs, rhs, atol=1e-11)


# ------------------------------------------------------- position maps ------
CW = [(128, 32), (64, 16), (16, 0), (12, 7), (10, 4), (4096, 1024)]


@pytest.mark.parametrize("c,w", CW)
def test_position_table_bounds_and_exact_regions(c, w):
    s = c - w
    L = min(4 * s + s // 2 + 3, 600)
    M = oracle.relative_position_table(L, c, w)
    i, j = np.tril_indices(L)
    m = M[i, j]
    rho = i // s - j // s
    # Every causal effective distance lies inside the pretrain window.
    assert m.min() >= 0 and m.max() <= c - 1
    # Intra-chunk: the exact, unscaled distance.
    assert np.array_equal(m[rho == 0], (i - j)[rho == 0])
    # Successive with the query inside the first w offsets: still exact.
    exact = (rho == 1) & (i % s < w)
    assert np.array_equal(m[exact], (i - j)[exact])
    # Everything else sees at least the local window.
    far = (rho >= 2) | ((rho == 1) & (i % s >= w))
    if far.any():
        assert m[far].min() >= w
    # Successive map is non-decreasing in the query offset for a fixed key.
    for jj in range(0, L, max(1, s // 3)):
        rows = np.arange(L)
        sel = (rows // s - jj // s) == 1
        if sel.sum() > 1:
            assert np.all(np.diff(M[rows[sel], jj]) >= 0)
    # Upper triangle is unused.
    assert np.all(M[np.triu_indices(L, 1)] == -1)


@pytest.mark.parametrize("c,w", CW)
def test_vectorised_maps_equal_bruteforce(c, w):
    s = c - w
    L = min(3 * s + 5, 400)
    M = oracle.relative_position_table(L, c, w)
    i, j = np.tril_indices(L)
    rho = oracle.relation(i, j, s)
    pi, ps, pe = oracle.query_positions(i, c, w)
    pq = np.where(rho == 0, pi, np.where(rho == 1, ps, pe))
    assert np.array_equal(pq - oracle.key_position(j, c, w), M[i, j])


def test_pages_printed_position_examples():
    with open(os.path.join(GOLDEN, "pages_position_examples.json")) as f:
        g = json.load(f)
    c = g["pretrain_length"]
    w = c - g["chunk_size"]
    for p in g["intra_pairs"]:
        i, j = p["i"], p["j"]
        rho = oracle.relation(i, j, c - w)
        assert rho == 0
        pq = oracle.query_positions(i, c, w)[0]
        assert pq - oracle.key_position(j, c, w) == p["effective_distance"] == p["raw_distance"]
    # The safety check over the causal half of a 16384-token horizon.  The
    # maximum is taken analytically per relation over all (i, j) with j <= i
    # (the full 16384^2 table would be 2 GiB).
    Lh = g["safety_invariant"]["seq_len"]
    s = c - w
    i = np.arange(Lh)
    pi, ps, pe = oracle.query_positions(i, c, w)
    worst = 0
    n = i // s
    # intra: max over keys j in [n*s, i] of pq - r(j) is pq - 0
    worst = max(worst, int((pi - 0).max()))
    has_prev = n >= 1
    worst = max(worst, int(ps[has_prev].max()))  # keys of the previous chunk, r(j) >= 0
    has_far = n >= 2
    worst = max(worst, int(pe[has_far].max()))
    assert worst <= g["safety_invariant"]["max_effective_distance_at_most"]


def test_remap_position_table_small():
    # c = 10, w = 4, s = 6.  Written out by hand from the readings.
    c, w = 10, 4
    t = np.arange(14)
    assert list(oracle.remap_positions(t, oracle.MAP_KEY, c, w)) == \
        [0, 1, 2, 3, 4, 5, 0, 1, 2, 3, 4, 5, 0, 1]
    assert list(oracle.remap_positions(t, oracle.MAP_Q_INTRA, c, w)) == \
        [0, 1, 2, 3, 4, 5, 0, 1, 2, 3, 4, 5, 0, 1]
    assert list(oracle.remap_positions(t, oracle.MAP_Q_SUCC, c, w)) == \
        [6, 7, 8, 9, 9, 9, 6, 7, 8, 9, 9, 9, 6, 7]
    assert list(oracle.remap_positions(t, oracle.MAP_Q_INTER, c, w)) == [9] * 14
    assert list(oracle.remap_positions(t + 3, oracle.MAP_PLAIN, c, w)) == list(t + 3)


# ---------------------------------------------------------- attention -------
def _sdpa_plain_rope(q, k, v, base, scale):
    """Plain RoPE causal attention via PyTorch's fp64 SDPA (the library routine)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    pos = np.arange(L)[None, :, None]
    qr = _rope_complex(q, pos, base)
    kr = _rope_complex(k, pos, base)
    G = Hq // Hkv
    kt = torch.from_numpy(kr).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    qt = torch.from_numpy(qr).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("c,w,L,Hq,Hkv,D", [(128, 32, 128, 2, 1, 64), (64, 16, 50, 4, 2, 32),
                                            (96, 48, 96, 1, 1, 16)])
def test_F1_equals_plain_rope_when_sequence_fits_pretrain_length(c, w, L, Hq, Hkv, D):
    q, k, v = inputs.prefill_inputs(1, L, Hq, Hkv, D, "f32", seed=7, qk_scale=2.0)
    scale = 1.0 / math.sqrt(D)
    O, _ = oracle.dca_prefill_ref(q, k, v, c, w, 10000.0, scale)
    want = _sdpa_plain_rope(q, k, v, 10000.0, scale)
    assert np.abs(O - want).max() < 1e-12


def test_F1_first_c_rows_of_a_long_sequence():
    c, w = 64, 16
    q, k, v = inputs.prefill_inputs(1, 200, 2, 2, 32, "f32", seed=3, qk_scale=2.0)
    rows = np.arange(c)
    O, _ = oracle.dca_prefill_ref(q, k, v, c, w, 10000.0, rows=rows)
    want = _sdpa_plain_rope(q[:, :c], k[:, :c], v[:, :c], 10000.0, 1 / math.sqrt(32))
    assert np.abs(O - want).max() < 1e-12
    # ... while later rows do differ from plain RoPE (the map is active).
    O2, _ = oracle.dca_prefill_ref(q, k, v, c, w, 10000.0, rows=[199])
    plain = _sdpa_plain_rope(q, k, v, 10000.0, 1 / math.sqrt(32))[:, 199:200]
    assert np.abs(O2 - plain).max() > 1e-3


@pytest.mark.parametrize("c,w,L,Hq,Hkv,D,a", [(32, 8, 150, 2, 1, 16, 2.0), (16, 0, 70, 1, 1, 8, 1.0),
                                              (12, 7, 61, 2, 2, 8, 2.0)])
def test_formA_equals_formB(c, w, L, Hq, Hkv, D, a):
    q, k, v = inputs.prefill_inputs(1, L, Hq, Hkv, D, "f32", seed=11, qk_scale=a)
    OA, LA = oracle.dca_prefill_ref(q, k, v, c, w, 10000.0)
    OB, LB = oracle.dca_prefill_formB(q, k, v, c, w, 10000.0)
    assert np.abs(OA - OB).max() < 1e-12
    assert np.abs(LA - LB).max() < 1e-12


def test_F3_softmax_rows_sum_to_one_and_constant_v():
    q, k, v = inputs.prefill_inputs(1, 100, 1, 1, 16, "f32", seed=5, qk_scale=3.0)
    _, _, P = oracle.dca_prefill_ref(q, k, v, 32, 8, 10000.0, return_probs=True)
    assert np.abs(P.sum(-1) - 1.0).max() < 1e-12
    assert np.all(P[0, 0][np.triu_indices(100, 1)] == 0)
    O, _ = oracle.dca_prefill_ref(q, k, torch.ones_like(v), 32, 8, 10000.0)
    assert np.abs(O - 1.0).max() < 1e-13


def test_LSE_is_log_of_partition_function():
    q, k, v = inputs.prefill_inputs(1, 40, 1, 1, 8, "f32", seed=9, qk_scale=2.0)
    c, w = 16, 4
    _, LSE = oracle.dca_prefill_ref(q, k, v, c, w, 10000.0)
    M = oracle.relative_position_table(40, c, w)
    qq, kk = np.asarray(q, float)[0, :, 0], np.asarray(k, float)[0, :, 0]
    for i in (0, 5, 17, 39):
        z = sum(math.exp(float(qq[i] @ _rope_complex(kk[j], -M[i, j], 1e4)) / math.sqrt(8))
                for j in range(i + 1))
        assert abs(LSE[0, 0, i] - math.log(z)) < 1e-12


def test_F4_inter_chunk_permutation_invariance():
    c, w = 64, 16
    s = c - w
    L = 6 * s
    q, k, v = inputs.prefill_inputs(1, L, 1, 1, 16, "f32", seed=21, qk_scale=2.0)
    rows = [5 * s, 5 * s + 3, 5 * s + w + 2, L - 1]   # queries in chunk 5
    O, _ = oracle.dca_prefill_ref(q, k, v, c, w, 10000.0, rows=rows)

    def swap(x, a, b):
        y = x.clone()
        y[:, a * s:(a + 1) * s], y[:, b * s:(b + 1) * s] = x[:, b * s:(b + 1) * s], x[:, a * s:(a + 1) * s]
        return y
    # Chunks 0 and 2 are both inter-chunk for every query of chunk 5.
    O2, _ = oracle.dca_prefill_ref(q, swap(k, 0, 2), swap(v, 0, 2), c, w, 10000.0, rows=rows)
    assert np.abs(O - O2).max() < 1e-12
    # Chunk 4 (successive) swapped with chunk 1 (inter) does change the output.
    O3, _ = oracle.dca_prefill_ref(q, swap(k, 1, 4), swap(v, 1, 4), c, w, 10000.0, rows=rows)
    assert np.abs(O - O3).max() > 1e-3


def test_F5_causality():
    q, k, v = inputs.prefill_inputs(1, 90, 1, 1, 16, "f32", seed=4, qk_scale=2.0)
    O, _ = oracle.dca_prefill_ref(q, k, v, 32, 8, 10000.0, rows=np.arange(50))
    k2, v2 = k.clone(), v.clone()
    k2[:, 50:] = 7.0
    v2[:, 50:] = -3.0
    O2, _ = oracle.dca_prefill_ref(q, k2, v2, 32, 8, 10000.0, rows=np.arange(50))
    assert np.abs(O - O2).max() == 0.0


def test_F6_gqa_equals_mha_with_repeated_kv():
    q, k, v = inputs.prefill_inputs(1, 80, 4, 2, 16, "f32", seed=8, qk_scale=2.0)
    O, L_ = oracle.dca_prefill_ref(q, k, v, 32, 8, 10000.0)
    O2, L2 = oracle.dca_prefill_ref(q, k.repeat_interleave(2, dim=2), v.repeat_interleave(2, dim=2),
                                    32, 8, 10000.0)
    assert np.abs(O - O2).max() == 0.0 and np.abs(L_ - L2).max() == 0.0
    # Head 1 reads KV head 0, head 2 reads KV head 1 (contiguous groups).
    O3, _ = oracle.dca_prefill_ref(q[:, :, 1:2], k[:, :, 0:1], v[:, :, 0:1], 32, 8, 10000.0)
    assert np.abs(O3[:, :, 0] - O[:, :, 1]).max() == 0.0


def test_F7_decode_equals_last_prefill_row():
    c, w = 32, 8
    L = 123
    q, k, v = inputs.prefill_inputs(2, L, 4, 2, 16, "f32", seed=12, qk_scale=2.0)
    O, LSE = oracle.dca_prefill_ref(q, k, v, c, w, 10000.0, rows=[L - 1])
    Od, Ld = oracle.dca_decode_ref(q[:, L - 1], k, v, c, w, 10000.0)
    assert np.abs(Od - O[:, 0]).max() < 1e-13
    assert np.abs(Ld - LSE[:, :, 0]).max() < 1e-13


# ------------------------------------------------------- planted keys -------
def planted_case(c, w, i, jstar, D=16, seed=0, target_logit=3.0):
    """All keys zero except k_{j*} = alpha R_{M*} q_i with M* the expected distance.

    Then the logit of j* is exactly target_logit, every other logit is 0, and
    O_i = (e^{T} v_{j*} + sum_{j <= i, j != j*} v_j) / (e^{T} + i) in closed form.
    """
    s = c - w
    rng = np.random.default_rng(seed)
    L = i + 1
    q = rng.standard_normal((1, L, 1, D))
    v = rng.standard_normal((1, L, 1, D))
    k = np.zeros((1, L, 1, D))
    rho = i // s - jstar // s
    if rho == 0 or (rho == 1 and i % s < w):
        Mstar = i - jstar                      # exact distance (pages + fact F1)
    else:
        Mstar = (c - 1) - (jstar % s)          # saturated query, chunk-local key
    scale = 1 / math.sqrt(D)
    alpha = target_logit / (scale * float(q[0, i, 0] @ q[0, i, 0]))
    k[0, jstar, 0] = alpha * _rope_complex(q[0, i, 0], Mstar, 1e4)
    e = math.exp(target_logit)
    want = (e * v[0, jstar, 0] + v[0, :L, 0].sum(0) - v[0, jstar, 0]) / (e + i)
    return q, k, v, want


PLANTED = {
    "intra": (64, 16, 100, 97),          # s = 48: i, j* both in chunk 2
    "succ_exact": (64, 16, 100, 60),     # r(i) = 4 < w
    "succ_saturated": (64, 16, 125, 60),  # r(i) = 29 >= w
    "inter": (64, 16, 200, 30),          # chunk 4 vs chunk 0
    "inter_tail": (128, 32, 511, 95),    # tiny-config geometry, last partial chunk
    "inter_far": (64, 16, 250, 100),     # chunk 5 vs chunk 2, key offset 4
}


@pytest.mark.parametrize("case", sorted(PLANTED))
def test_planted_key_closed_form(case):
    c, w, i, jstar = PLANTED[case]
    q, k, v, want = planted_case(c, w, i, jstar)
    O, _ = oracle.dca_prefill_ref(q, k, v, c, w, 1e4, rows=[i])
    assert np.abs(O[0, 0, 0] - want).max() < 1e-12
    Od, _ = oracle.dca_decode_ref(q[:, i], k, v, c, w, 1e4)
    assert np.abs(Od[0, 0] - want).max() < 1e-12


# ------------------------------------------- planted oracle mistakes --------
def _mutants():
    good = ref.query_positions

    def succ_as_inter(i, c, w):
        a, b, e = good(i, c, w)
        return a, e, e

    def succ_unsaturated(i, c, w):
        a, b, e = good(i, c, w)
        return a, (c - w) + a, e

    def inter_off_by_one(i, c, w):
        a, b, e = good(i, c, w)
        return a, b, e - 1

    def intra_absolute(i, c, w):
        a, b, e = good(i, c, w)
        return np.asarray(i, dtype=np.int64), b, e
    return {"succ_as_inter": succ_as_inter, "succ_unsaturated": succ_unsaturated,
            "inter_off_by_one": inter_off_by_one, "intra_absolute": intra_absolute}


@pytest.mark.parametrize("mutant", sorted(_mutants()))
def test_pins_catch_planted_oracle_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(ref, "query_positions", _mutants()[mutant])
    caught = []
    for case, (c, w, i, jstar) in PLANTED.items():
        q, k, v, want = planted_case(c, w, i, jstar)
        O, _ = oracle.dca_prefill_ref(q, k, v, c, w, 1e4, rows=[i])
        if np.abs(O[0, 0, 0] - want).max() > 1e-6:
            caught.append(case)
    assert caught, f"mutant {mutant} survived every planted-key pin"


def test_pins_catch_wrong_key_position(monkeypatch):
    monkeypatch.setattr(ref, "key_position", lambda j, c, w: np.asarray(j, dtype=np.int64) % c)
    c, w, i, jstar = PLANTED["inter_far"]
    q, k, v, want = planted_case(c, w, i, jstar)
    O, _ = oracle.dca_prefill_ref(q, k, v, c, w, 1e4, rows=[i])
    assert np.abs(O[0, 0, 0] - want).max() > 1e-6


def test_pins_catch_wrong_pairing(monkeypatch):
    def interleaved(x, pos, base):  # adjacent-pair convention instead of rotate-half
        x = ref._f64(x)
        D = x.shape[-1]
        ang = np.asarray(pos, dtype=np.float64)[..., None] * ref.rope_inv_freq(D, base)
        x1, x2 = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = x1 * np.cos(ang) - x2 * np.sin(ang)
        out[..., 1::2] = x2 * np.cos(ang) + x1 * np.sin(ang)
        return out
    monkeypatch.setattr(ref, "rope_rotate", interleaved)
    monkeypatch.setattr(oracle, "rope_rotate", interleaved)
    with pytest.raises(AssertionError):
        test_rope_closed_form_d4_pairing_and_frequencies()


# ------------------------------------------------ chunked prefill (prefix) ---
@pytest.mark.parametrize("pos0,Lq", [(0, 50), (37, 40), (64, 59), (100, 23)])
def test_chunk_rows_equal_full_prefill_rows(pos0, Lq):
    # Prefix consistency: the chunk's rows are rows pos0.. of the whole prompt.
    c, w = 32, 8
    L = pos0 + Lq
    q, k, v = inputs.prefill_inputs(2, L, 4, 2, 16, "f32", seed=13, qk_scale=2.0)
    O, LSE = oracle.dca_prefill_ref(q, k, v, c, w, 10000.0, rows=np.arange(pos0, L))
    Oc, Lc = oracle.dca_prefill_chunk_ref(q[:, pos0:], k, v, pos0, c, w, 10000.0)
    assert np.abs(Oc - O).max() < 1e-13
    assert np.abs(Lc - LSE).max() < 1e-13


def test_chunks_concatenate_to_the_full_prefill():
    c, w = 24, 6
    L = 130
    q, k, v = inputs.prefill_inputs(1, L, 2, 1, 8, "f32", seed=14, qk_scale=2.0)
    O, _ = oracle.dca_prefill_ref(q, k, v, c, w, 10000.0)
    parts = [oracle.dca_prefill_chunk_ref(q[:, a:b], k[:, :b], v[:, :b], a, c, w, 10000.0)[0]
             for a, b in ((0, 40), (40, 41), (41, 100), (100, 130))]
    assert np.abs(np.concatenate(parts, axis=1) - O).max() < 1e-13


def test_single_row_chunk_is_decode_and_ragged_rows_are_independent():
    c, w = 32, 8
    q, k, v = inputs.prefill_inputs(2, 90, 4, 2, 16, "f32", seed=15, qk_scale=2.0)
    Od, Ld = oracle.dca_decode_ref(q[:, 89], k, v, c, w, 10000.0)
    Oc, Lc = oracle.dca_prefill_chunk_ref(q[:, 89:90], k, v, 89, c, w, 10000.0)
    assert np.abs(Oc[:, 0] - Od).max() < 1e-13 and np.abs(Lc[:, :, 0] - Ld).max() < 1e-13
    # ragged: sequence 1 has its chunk at a different offset and fewer rows
    pos0, q_len = [60, 45], [30, 12]
    qc = torch.zeros(2, 30, 4, 16, dtype=torch.float32)
    qc[0] = q[0, 60:90]
    qc[1, :12] = q[1, 45:57]
    Or, Lr = oracle.dca_prefill_chunk_ref(qc, k, v, pos0, c, w, 10000.0, q_len=q_len)
    O0, _ = oracle.dca_prefill_ref(q[0:1], k[0:1], v[0:1], c, w, 10000.0, rows=np.arange(60, 90))
    O1, _ = oracle.dca_prefill_ref(q[1:2], k[1:2], v[1:2], c, w, 10000.0, rows=np.arange(45, 57))
    assert np.abs(Or[0] - O0[0]).max() < 1e-13
    assert np.abs(Or[1, :12] - O1[0]).max() < 1e-13
    assert np.all(Or[1, 12:] == 0) and np.all(np.isneginf(Lr[1, :, 12:]))
