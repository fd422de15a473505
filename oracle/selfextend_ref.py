"""Plain fp64 CPU oracle for SelfExtend-style grouped / neighbor attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It imports nothing
from the HIP library or its Python binding; like the DCA oracle beside it, every
function is the definition written out in fp64 NumPy.

Source: "LLM Maybe LongLM: Self-Extend LLM Context Window Without Tuning"
(abstract).  The method builds two levels of attention out of the model's own
self-attention: *grouped* attention for tokens that are far apart and
*neighbor* attention for tokens inside a chosen range, without any training.

The abstract gives no formulas.  Readings (listed in the design notes):

* neighbor pairs are those with distance i - j < W (the neighbor window); they
  keep ordinary RoPE positions, key at j and query at i, so their relative
  position is exactly i - j;
* grouped pairs (i - j >= W) place key j at floor(j / G) (G = group size: G
  consecutive keys share one position) and query i at
  floor(i / G) + W - floor(W / G); the shift makes the grouped relative
  position continue the neighbor one at the window edge (for i, j multiples
  of G at distance W it is exactly W) and keeps it >= W for every grouped pair;
* causal with the diagonal kept; RoPE, the softmax scale, natural-log LSE and
  GQA head mapping exactly as in the DCA oracle.

Pins (tests): G = 1 and W >= L both reduce to plain RoPE attention (checked
against fp64 scaled_dot_product_attention); form A equals the brute-force
form B; the relative-position table satisfies M = i - j for neighbor pairs,
M >= W for grouped pairs and depends on j only through floor(j / G) there
(swapping two keys of one group leaves a row unchanged); a planted key gives
the closed-form output in both relations.  For G > 1 and W < L no printed
value exists: beyond those invariants the exact constants (the shift above)
are a reading, so the SelfExtend outputs are "parity unpinned" for the shift.
"""
from __future__ import annotations

import numpy as np

from .dca_ref import _f64, _kv_head, _softmax_rows, rope_rotate

MAP_SE_KEY_GROUPED = 5   # P = floor(t / G)
MAP_SE_Q_GROUPED = 6     # P = floor(t / G) + W - floor(W / G)

NEIGHBOR = 0
GROUPED = 1


def _check(G: int, W: int) -> None:
    if G < 1 or W < 0:
        raise ValueError(f"need group >= 1 and window >= 0, got G={G} W={W}")


def se_relation(i, j, W: int):
    """0 (neighbor) when i - j < W, else 1 (grouped); for causal pairs j <= i."""
    d = np.asarray(i, dtype=np.int64) - np.asarray(j, dtype=np.int64)
    return np.where(d < W, NEIGHBOR, GROUPED)


def se_key_position(j, G: int, rel):
    """Key position: j for neighbor pairs, floor(j / G) for grouped pairs."""
    j = np.asarray(j, dtype=np.int64)
    return np.where(np.asarray(rel) == GROUPED, j // G, j)


def se_query_position(i, G: int, W: int, rel):
    """Query position: i for neighbor pairs, floor(i/G) + W - floor(W/G) for grouped."""
    _check(G, W)
    i = np.asarray(i, dtype=np.int64)
    return np.where(np.asarray(rel) == GROUPED, i // G + W - W // G, i)


def se_relative_position_table(L: int, G: int, W: int) -> np.ndarray:
    """Brute-force M[i][j] = P_q - P_k for every causal pair, -1 elsewhere.

    Python loops with the rules written out per pair (tiny L only): the second
    formulation the vectorised maps and the kernels' maps are checked against.
    """
    _check(G, W)
    M = np.full((L, L), -1, dtype=np.int64)
    for i in range(L):
        for j in range(i + 1):
            if i - j < W:
                pq, pk = i, j
            else:
                pq, pk = i // G + W - W // G, j // G
            M[i, j] = pq - pk
    return M


def se_remap_positions(t, map_kind: int, G: int, W: int):
    """Rotation position of the two grouped remap maps for token position t."""
    _check(G, W)
    t = np.asarray(t, dtype=np.int64)
    if map_kind == MAP_SE_KEY_GROUPED:
        return t // G
    if map_kind == MAP_SE_Q_GROUPED:
        return t // G + W - W // G
    raise ValueError(f"unknown SelfExtend map kind {map_kind}")


def se_rope_remap_ref(x, pos0: int, map_kind: int, G: int, W: int, base: float) -> np.ndarray:
    """x: [B, L, H, D]; token t sits at pos0 + t; rotate by the grouped map's position."""
    x = _f64(x)
    pos = se_remap_positions(pos0 + np.arange(x.shape[1]), map_kind, G, W)
    return rope_rotate(x, pos[None, :, None], base)


def selfextend_prefill_ref(q, k, v, G: int, W: int, base: float = 10000.0,
                           sm_scale: float | None = None, rows=None, heads=None):
    """Form A: causal SelfExtend prefill, evaluated row by row.

    q: [B, L, Hq, D] raw; k, v: [B, L, Hkv, D] raw.  For query row i the keys
    j in (i - W, i] use the neighbor positions (query i, key j); the keys
    j <= i - W use the grouped positions (query floor(i/G) + W - floor(W/G),
    key floor(j/G)).  Returns O [B, rows, heads, D] and LSE [B, heads, rows].
    """
    _check(G, W)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    O = np.zeros((B, len(rows), len(heads), D))
    LSE = np.zeros((B, len(heads), len(rows)))
    jj = np.arange(L)
    for b in range(B):
        cache = {}
        for hi, h in enumerate(heads):
            g = _kv_head(int(h), Hq, Hkv)
            if g not in cache:   # the two key rotations of every key
                cache[g] = (rope_rotate(k[b, :, g], se_key_position(jj, G, NEIGHBOR), base),
                            rope_rotate(k[b, :, g], se_key_position(jj, G, GROUPED), base))
            k_nb, k_gr = cache[g]
            for ri, i in enumerate(rows):
                i = int(i)
                rel = se_relation(i, jj[: i + 1], W)
                S = np.empty(i + 1)
                for r_kind, khat in ((NEIGHBOR, k_nb), (GROUPED, k_gr)):
                    sel = rel == r_kind
                    if sel.any():
                        qv = rope_rotate(q[b, i, h], se_query_position(i, G, W, r_kind), base)
                        S[sel] = scale * (khat[: i + 1][sel] @ qv)
                o, lse = _softmax_rows(S[None, :], v[b, : i + 1, g])
                O[b, ri, hi] = o[0]
                LSE[b, hi, ri] = lse[0]
    return O, LSE


def selfextend_prefill_formB(q, k, v, G: int, W: int, base: float = 10000.0,
                             sm_scale: float | None = None):
    """Form B (tiny sizes): scores from the brute-force relative-position table,
    S_ij = sm_scale * q_i . (R_{-M_ij} k_j) on the raw q and k."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    M = se_relative_position_table(L, G, W)
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


def selfextend_decode_ref(q, k_raw, v, kv_len, G: int, W: int, base: float = 10000.0,
                          sm_scale: float | None = None):
    """Decode under the SelfExtend map: sequence b's new token is row
    kv_len[b] - 1 of the prefill definition over its first kv_len[b] cached
    keys.  q: [B, Hq, D] raw; k_raw, v: [B, cache_len, Hkv, D] raw.
    Returns O [B, Hq, D] and LSE [B, Hq]."""
    _check(G, W)
    q = _f64(q)
    B, Hq, D = q.shape
    Hkv = k_raw.shape[2]
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    O = np.zeros((B, Hq, D))
    LSE = np.zeros((B, Hq))
    for b in range(B):
        n = int(kv_len[b])
        i = n - 1
        jj = np.arange(n)
        rel = se_relation(i, jj, W)
        for g in range(Hkv):
            kb = _f64(k_raw[b, :n, g])
            k_nb = rope_rotate(kb, se_key_position(jj, G, NEIGHBOR), base)
            k_gr = rope_rotate(kb, se_key_position(jj, G, GROUPED), base)
            vb = _f64(v[b, :n, g])
            for h in range(Hq):
                if _kv_head(h, Hq, Hkv) != g:
                    continue
                S = np.empty(n)
                for r_kind, khat in ((NEIGHBOR, k_nb), (GROUPED, k_gr)):
                    sel = rel == r_kind
                    if sel.any():
                        qv = rope_rotate(q[b, h], se_query_position(i, G, W, r_kind), base)
                        S[sel] = scale * (khat[sel] @ qv)
                o, lse = _softmax_rows(S[None, :], vb)
                O[b, h] = o[0]
                LSE[b, h] = lse[0]
    return O, LSE
