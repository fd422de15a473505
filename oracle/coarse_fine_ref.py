"""Plain fp64 CPU oracle for the DCA guide's coarse / fine position map.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It imports nothing
from the HIP library or its Python binding.

Source: "Dual-Chunk Attention: Training-Free 100k+ Context Guide", the
"Inter-Chunk Attention" section and "Deep Dive" sub-section "1. Successive
Chunk Smoothing" (and the "End-to-End Implementation" script built from them).
With chunk size C, chunk index c_x = floor(x / C), offset o_x = x mod C and
kappa = L_target / L_train (the guide calls it s; renamed to avoid the chunk
size symbol), the effective distance of a causal pair (i >= j) is

  same chunk (c_i = c_j):       i - j
  chunks >= 2 apart:            (c_i - c_j) * C / kappa + (o_i - o_j)
  adjacent chunks:              (1 - lambda) (i - j) + lambda * (inter value),
                                lambda = o_i / C.

Distances are real numbers; the rotation angle of a pair is its distance
times theta_k.  No reading is needed beyond the DCA oracle's (rotate-half
RoPE, softmax scale, causal diagonal, GQA).  This map can go negative
(e.g. -383 at (1024, 511) with C 512 and kappa 8) and past L_train at
L = L_target; it is built as the guide states it, not clamped.

Two formulations: form B writes the three formulas per pair
(``coarse_fine_distance_table``); form A factors every distance into a query
position minus a key position, the way the kernels compute it:

  key:   plain j (same or adjacent chunk), scaled c_j * C / kappa + o_j (inter)
  query: intra i;  successive i - o_i (1 - 1/kappa);  inter c_i * C / kappa + o_i

(every key of an adjacent-chunk pair lies in chunk c_i - 1, which is what lets
the successive ramp become one query position).
"""
from __future__ import annotations

import numpy as np

from .dca_ref import _f64, _kv_head, _softmax_rows, rope_rotate


def _kappa(train_len: int, target_len: int) -> float:
    if train_len < 1 or target_len < 1:
        raise ValueError("training and target lengths must be positive")
    return float(target_len) / float(train_len)


def coarse_fine_distance_table(L: int, C: int, train_len: int, target_len: int) -> np.ndarray:
    """Form B positions: the guide's effective distance per causal pair (Python
    loops over the three formulas; tiny L only).  NaN above the diagonal."""
    if C < 1:
        raise ValueError("chunk size must be positive")
    kappa = _kappa(train_len, target_len)
    M = np.full((L, L), np.nan)
    for i in range(L):
        ci, oi = divmod(i, C)
        for j in range(i + 1):
            cj, oj = divmod(j, C)
            inter = (ci - cj) * C / kappa + (oi - oj)
            if ci == cj:
                M[i, j] = i - j
            elif ci == cj + 1:
                lam = oi / C
                M[i, j] = (1.0 - lam) * (i - j) + lam * inter
            else:
                M[i, j] = inter
    return M


def coarse_fine_positions(i, C: int, train_len: int, target_len: int):
    """Form A query positions (intra, successive, inter) of query i."""
    kappa = _kappa(train_len, target_len)
    i = np.asarray(i, dtype=np.float64)
    c, o = np.floor(i / C), np.mod(i, C)
    return i, i - o * (1.0 - 1.0 / kappa), c * C / kappa + o


def coarse_fine_key_positions(j, C: int, train_len: int, target_len: int):
    """Form A key positions: (plain, scaled) of key j."""
    kappa = _kappa(train_len, target_len)
    j = np.asarray(j, dtype=np.float64)
    return j, np.floor(j / C) * C / kappa + np.mod(j, C)


def coarse_fine_prefill_ref(q, k, v, C: int, train_len: int, target_len: int, base: float = 10000.0,
                            sm_scale: float | None = None, rows=None, heads=None):
    """Form A: causal prefill under the coarse / fine map, row by row.

    q: [B, L, Hq, D] raw; k, v: [B, L, Hkv, D] raw.  Keys in the query's chunk
    and the one before use the plain key rotation, older chunks the scaled one;
    the query takes its intra / successive / inter position accordingly.
    Returns O [B, rows, heads, D] and LSE [B, heads, rows].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    O = np.zeros((B, len(rows), len(heads), D))
    LSE = np.zeros((B, len(heads), len(rows)))
    kp_plain, kp_scaled = coarse_fine_key_positions(np.arange(L), C, train_len, target_len)
    for b in range(B):
        cache = {}
        for hi, h in enumerate(heads):
            g = _kv_head(int(h), Hq, Hkv)
            if g not in cache:
                cache[g] = (rope_rotate(k[b, :, g], kp_plain, base), rope_rotate(k[b, :, g], kp_scaled, base))
            k_pl, k_sc = cache[g]
            for ri, i in enumerate(rows):
                i = int(i)
                n = i // C
                p_intra, p_succ, p_inter = coarse_fine_positions(i, C, train_len, target_len)
                S = np.empty(i + 1)
                for lo, hi_, pq, khat in ((n * C, i + 1, p_intra, k_pl), ((n - 1) * C, n * C, p_succ, k_pl),
                                          (0, (n - 1) * C, p_inter, k_sc)):
                    lo = max(lo, 0)
                    if hi_ <= lo:
                        continue
                    S[lo:hi_] = scale * (khat[lo:hi_] @ rope_rotate(q[b, i, h], pq, base))
                o, lse = _softmax_rows(S[None, :], v[b, : i + 1, g])
                O[b, ri, hi] = o[0]
                LSE[b, hi, ri] = lse[0]
    return O, LSE


def coarse_fine_prefill_formB(q, k, v, C: int, train_len: int, target_len: int, base: float = 10000.0,
                              sm_scale: float | None = None):
    """Form B (tiny sizes): S_ij = sm_scale * q_i . (R_{-M_ij} k_j) with M from the
    guide's three distance formulas, on the raw q and k."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    M = coarse_fine_distance_table(L, C, train_len, target_len)
    O = np.zeros((B, L, Hq, D))
    LSE = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            for i in range(L):
                krot = rope_rotate(k[b, : i + 1, g], -M[i, : i + 1], base)
                o, lse = _softmax_rows((scale * (krot @ q[b, i, h]))[None, :], v[b, : i + 1, g])
                O[b, i, h] = o[0]
                LSE[b, h, i] = lse[0]
    return O, LSE


def coarse_fine_key_remap_ref(x, pos0: int, C: int, train_len: int, target_len: int,
                              base: float = 10000.0) -> np.ndarray:
    """Keys rotated at their coarse-scaled positions floor(p/C) C / kappa + p mod C
    (the rotation every key takes in pairs two or more chunks apart), for the
    rows of x [B, L, H, D] at positions pos0 .. pos0 + L - 1."""
    x = _f64(x)
    L = x.shape[1]
    _, p = coarse_fine_key_positions(pos0 + np.arange(L), C, train_len, target_len)
    return rope_rotate(x, p[None, :, None], base)


def coarse_fine_decode_ref(q, k_raw, v, kv_len, C: int, train_len: int, target_len: int,
                           base: float = 10000.0, sm_scale: float | None = None):
    """Decode under the coarse / fine map: sequence b's new token is row
    kv_len[b] - 1 of the prefill definition over its first kv_len[b] keys.
    q: [B, Hq, D] raw; k_raw, v: [B, cache_len, Hkv, D] raw.
    Returns O [B, Hq, D] and LSE [B, Hq]."""
    q = _f64(q)
    B, Hq, D = q.shape
    Hkv = k_raw.shape[2]
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    O = np.zeros((B, Hq, D))
    LSE = np.zeros((B, Hq))
    for b in range(B):
        n = int(kv_len[b])
        i = n - 1
        c = i // C
        kp_plain, kp_scaled = coarse_fine_key_positions(np.arange(n), C, train_len, target_len)
        p_intra, p_succ, p_inter = coarse_fine_positions(i, C, train_len, target_len)
        for g in range(Hkv):
            kb = _f64(k_raw[b, :n, g])
            k_pl, k_sc = rope_rotate(kb, kp_plain, base), rope_rotate(kb, kp_scaled, base)
            vb = _f64(v[b, :n, g])
            for h in range(Hq):
                if _kv_head(h, Hq, Hkv) != g:
                    continue
                S = np.empty(n)
                for lo, hi_, pq, khat in ((c * C, n, p_intra, k_pl), ((c - 1) * C, c * C, p_succ, k_pl),
                                          (0, (c - 1) * C, p_inter, k_sc)):
                    lo = max(lo, 0)
                    if hi_ <= lo:
                        continue
                    S[lo:hi_] = scale * (khat[lo:hi_] @ rope_rotate(q[b, h], pq, base))
                o, lse = _softmax_rows(S[None, :], vb)
                O[b, h] = o[0]
                LSE[b, h] = lse[0]
    return O, LSE
