"""Plain fp64 CPU oracle for training-free Dual Chunk Attention (DCA).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It is slow on
purpose: every function is the definition written out in fp64 NumPy, with no
tiling, fusion or reordering beyond what the definition states.  It imports
nothing from the HIP library or its Python binding.

Sources (cited by page title and section):

* "Dual-Chunk Attention: Training-Free 100k+ Context Guide" (aifetchly blog),
  referred to below as *the DCA guide*:
    - "The Problem" section: the RoPE score identity q_i^T k_j =
      x_i^T W_Q^T R_{Theta, j-i} W_K x_j, i.e. a score depends only on the
      relative position, with angles (i - j) * theta_k per rotary pair.
    - "The Architecture" taxonomy box and its sub-sections "1. Intra-Chunk
      Attention" and "2. Inter-Chunk Attention": the sequence is cut into
      fixed-size chunks; the relation of a pair is decided by the chunk-index
      difference (0 = intra, 1 = successive, >= 2 = inter); intra pairs keep
      their true distance with no scaling; inter pairs keep the fine offset inside
      the key's chunk, and their distance stays below the pretrain length.
    - "Deep Dive", sub-section "1. Successive Chunk Smoothing": successive
      pairs see the plain local distance near the chunk edge and move
      continuously toward the inter-chunk value deeper into the chunk.
    - "End-to-End Implementation" script: causal pairs are those with i >= j
      (the diagonal included), and every causal pair's effective distance is
      bounded by the pretrain length.
* "LLM Maybe LongLM: Self-Extend LLM Context Window Without Tuning" code
  entry names ``rotate_half`` / ``apply_rotary_pos_emb`` / ``repeat_kv``:
  the rotate-half RoPE pairing and contiguous GQA head groups.

Readings taken where the pages are silent or contradict one another (each is
listed in the repository's design notes):

* chunk size s = c - w, with c the pretrain length and w the local window;
* key position P_k(j) = j mod s (the fine offset inside the key's chunk);
* query position by relation rho = floor(i/s) - floor(j/s):
    rho = 0 (intra):       P_q = i mod s
    rho = 1 (successive):  P_q = min(s + (i mod s), c - 1)
    rho >= 2 (inter):      P_q = c - 1
  so the effective relative position M = P_q - P_k always lies in [0, c-1],
  equals i - j exactly whenever the sequence fits the pretrain length, and is
  continuous where the successive map saturates;
* RoPE: theta_k = base^(-2k/D), pairing (k, k + D/2) ("rotate half");
* softmax scale sm_scale (default 1/sqrt(D)), natural-log LSE;
* GQA: query head h reads KV head floor(h * Hkv / Hq).

The functions take NumPy or torch arrays of any float dtype; values are cast
exactly to fp64 and no intermediate rounding happens.
"""
from __future__ import annotations

import numpy as np

MAP_KEY = 0
MAP_Q_INTRA = 1
MAP_Q_SUCC = 2
MAP_Q_INTER = 3
MAP_PLAIN = 4


def _f64(x) -> np.ndarray:
    """Exact cast to fp64 (torch bf16/fp32 tensors go through fp32, which is exact)."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    return np.asarray(x, dtype=np.float64)


def chunk_size(c: int, w: int) -> int:
    """Chunk size s = c - w (pretrain length minus local window)."""
    if not (0 <= w < c):
        raise ValueError(f"need 0 <= w < c, got c={c} w={w}")
    return c - w


# --------------------------------------------------------------------------
# RoPE ("The Problem" section of the DCA guide; rotate-half pairing from the
# SelfExtend code entry names)
# --------------------------------------------------------------------------
def rope_inv_freq(D: int, base: float) -> np.ndarray:
    """theta_k = base^(-2k/D) for k in [0, D/2), in fp64."""
    if D % 2:
        raise ValueError("head dim must be even")
    k = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * k / D)


def rope_rotate(x, pos, base: float) -> np.ndarray:
    """Rotate the last axis of ``x`` by position ``pos`` (rotate-half pairing).

    The pair (x[k], x[k + D/2]) is turned by the angle pos * theta_k:
        (x_k, x_{k+D/2}) -> (x_k cos a - x_{k+D/2} sin a,
                             x_{k+D/2} cos a + x_k sin a).
    ``pos`` broadcasts against ``x.shape[:-1]``.  Angles are fp64.
    """
    x = _f64(x)
    D = x.shape[-1]
    half = D // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(D, base)
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


# --------------------------------------------------------------------------
# DCA position maps ("The Architecture" box, intra / inter / successive
# sub-sections of the DCA guide, under the readings in the module docstring)
# --------------------------------------------------------------------------
def key_position(j, c: int, w: int):
    """P_k(j) = j mod s: the fine offset of key j inside its chunk."""
    s = chunk_size(c, w)
    return np.asarray(j, dtype=np.int64) % s


def query_positions(i, c: int, w: int):
    """(P_intra, P_succ, P_inter) of query i.

    intra:       i mod s                 (unscaled, same chunk)
    successive:  min(s + (i mod s), c-1) (exact distance until it saturates)
    inter:       c - 1                   (constant; keeps M inside [w, c-1])
    """
    s = chunk_size(c, w)
    i = np.asarray(i, dtype=np.int64)
    r = i % s
    return r, np.minimum(s + r, c - 1), np.full_like(r, c - 1)


def relation(i, j, s: int):
    """rho(i, j) = floor(i/s) - floor(j/s): 0 intra, 1 successive, >=2 inter."""
    return np.asarray(i, dtype=np.int64) // s - np.asarray(j, dtype=np.int64) // s


def relative_position_table(L: int, c: int, w: int) -> np.ndarray:
    """Brute-force M[i][j] = P_q - P_k for every causal pair (j <= i), -1 elsewhere.

    Written with explicit per-pair rules and Python loops (tiny L only); it is
    the second formulation the vectorised maps are checked against.
    """
    s = chunk_size(c, w)
    M = np.full((L, L), -1, dtype=np.int64)
    for i in range(L):
        ni, ri = divmod(i, s)
        for j in range(i + 1):
            nj, rj = divmod(j, s)
            if ni == nj:
                pq = ri
            elif ni == nj + 1:
                pq = s + ri if s + ri < c else c - 1
            else:
                pq = c - 1
            M[i, j] = pq - rj
    return M


def remap_positions(t, map_kind: int, c: int, w: int):
    """Rotation position used by the remap operation for token position t."""
    t = np.asarray(t, dtype=np.int64)
    if map_kind == MAP_PLAIN:
        return t
    if map_kind == MAP_KEY:
        return key_position(t, c, w)
    p_intra, p_succ, p_inter = query_positions(t, c, w)
    if map_kind == MAP_Q_INTRA:
        return p_intra
    if map_kind == MAP_Q_SUCC:
        return p_succ
    if map_kind == MAP_Q_INTER:
        return p_inter
    raise ValueError(f"unknown map kind {map_kind}")


def rope_remap_ref(x, pos0: int, map_kind: int, c: int, w: int, base: float) -> np.ndarray:
    """x: [B, L, H, D]; token t sits at position pos0 + t; rotate by the map's position."""
    x = _f64(x)
    L = x.shape[1]
    pos = remap_positions(pos0 + np.arange(L), map_kind, c, w)
    return rope_rotate(x, pos[None, :, None], base)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------
def _softmax_rows(S: np.ndarray, V: np.ndarray):
    """Row softmax with max subtraction; returns (P @ V, natural-log LSE)."""
    m = S.max(axis=-1, keepdims=True)
    e = np.exp(S - m)
    l = e.sum(axis=-1, keepdims=True)
    O = (e / l) @ V
    return O, (m + np.log(l))[..., 0]


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return (h * Hkv) // Hq


def dca_prefill_ref(q, k, v, c: int, w: int, base: float = 10000.0,
                    sm_scale: float | None = None, rows=None, heads=None,
                    return_probs: bool = False):
    """Form A: DCA causal prefill attention, evaluated row by row.

    q: [B, L, Hq, D] raw (pre-RoPE); k, v: [B, L, Hkv, D] raw.
    rows: query indices to evaluate (default all); heads: query heads.
    Returns O [B, len(rows), len(heads), D] and LSE [B, len(heads), len(rows)]
    (and the probability rows [B, heads, rows, L] when return_probs).

    For each query row i in chunk n = floor(i/s), the keys in chunk n use the
    intra variant of q_i, keys in chunk n-1 the successive variant and keys in
    chunks <= n-2 the inter variant; keys are rotated at j mod s; keys j > i
    are masked (causal, diagonal kept).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    s = chunk_size(c, w)
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    O = np.zeros((B, len(rows), len(heads), D))
    LSE = np.zeros((B, len(heads), len(rows)))
    probs = np.zeros((B, len(heads), len(rows), L)) if return_probs else None
    kpos = key_position(np.arange(L), c, w)
    for b in range(B):
        khat_cache = {}
        for hi, h in enumerate(heads):
            g = _kv_head(int(h), Hq, Hkv)
            if g not in khat_cache:
                khat_cache[g] = rope_rotate(k[b, :, g], kpos, base)
            khat, vg = khat_cache[g], v[b, :, g]
            for ri, i in enumerate(rows):
                i = int(i)
                n = i // s
                p_intra, p_succ, p_inter = query_positions(i, c, w)
                S = np.empty(i + 1)
                bounds = (
                    (n * s, i + 1, p_intra),           # same chunk
                    ((n - 1) * s, n * s, p_succ),       # previous chunk
                    (0, (n - 1) * s, p_inter),          # chunks <= n-2
                )
                for lo, hi_, pq in bounds:
                    lo = max(lo, 0)
                    if hi_ <= lo:
                        continue
                    qv = rope_rotate(q[b, i, h], pq, base)
                    S[lo:hi_] = scale * (khat[lo:hi_] @ qv)
                o, lse = _softmax_rows(S[None, :], vg[: i + 1])
                O[b, ri, hi] = o[0]
                LSE[b, hi, ri] = lse[0]
                if return_probs:
                    P = np.exp(S - lse[0])
                    probs[b, hi, ri, : i + 1] = P
    if return_probs:
        return O, LSE, probs
    return O, LSE


def dca_prefill_formB(q, k, v, c: int, w: int, base: float = 10000.0,
                      sm_scale: float | None = None):
    """Form B (tiny sizes): scores from the brute-force relative-position table.

    S_ij = sm_scale * q_i . (R_{-M_ij} k_j), using <R_a q, R_b k> = q^T R_{b-a} k,
    which is the RoPE relative-position identity of the DCA guide's "Problem"
    section.  Raw (unrotated) q is used, so no absolute position enters.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    M = relative_position_table(L, c, w)
    O = np.zeros((B, L, Hq, D))
    LSE = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            for i in range(L):
                krot = rope_rotate(k[b, : i + 1, g], -M[i, : i + 1], base)
                S = scale * (krot @ q[b, i, h])
                o, lse = _softmax_rows(S[None, :], v[b, : i + 1, g])
                O[b, i, h] = o[0]
                LSE[b, h, i] = lse[0]
    return O, LSE


def dca_decode_ref(q, k_raw, v, c: int, w: int, base: float = 10000.0,
                   sm_scale: float | None = None, batches=None, heads=None):
    """One new query token per sequence against a KV cache.

    q: [B, Hq, D] raw; k_raw: [B, kv_len, Hkv, D] *unrotated* keys; v likewise.
    The query sits at position kv_len - 1 (the cache includes the new token),
    so this is row kv_len - 1 of the prefill definition.
    Returns O [len(batches), len(heads), D] and LSE [len(batches), len(heads)].
    """
    q = _f64(q)
    B, Hq, D = q.shape
    kv_len, Hkv = k_raw.shape[1], k_raw.shape[2]
    s = chunk_size(c, w)
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    batches = np.arange(B) if batches is None else np.asarray(batches)
    heads = np.arange(Hq) if heads is None else np.asarray(heads)
    i = kv_len - 1
    n = i // s
    p_intra, p_succ, p_inter = query_positions(i, c, w)
    kpos = key_position(np.arange(kv_len), c, w)
    O = np.zeros((len(batches), len(heads), D))
    LSE = np.zeros((len(batches), len(heads)))
    for bi, b in enumerate(batches):
        cache = {}
        for hi, h in enumerate(heads):
            g = _kv_head(int(h), Hq, Hkv)
            if g not in cache:
                cache[g] = (rope_rotate(_f64(k_raw[int(b), :, g]), kpos, base),
                            _f64(v[int(b), :, g]))
            khat, vg = cache[g]
            S = np.empty(kv_len)
            for lo, hi_, pq in ((n * s, kv_len, p_intra), ((n - 1) * s, n * s, p_succ),
                                (0, (n - 1) * s, p_inter)):
                lo = max(lo, 0)
                if hi_ <= lo:
                    continue
                S[lo:hi_] = scale * (khat[lo:hi_] @ rope_rotate(q[int(b), int(h)], pq, base))
            o, lse = _softmax_rows(S[None, :], vg)
            O[bi, hi] = o[0]
            LSE[bi, hi] = lse[0]
    return O, LSE


def dca_prefill_chunk_ref(q, k_raw, v, pos0, c: int, w: int, base: float = 10000.0,
                          sm_scale: float | None = None, q_len=None, rows=None, heads=None):
    """Chunked prefill over a KV prefix: the new tokens of one chunk per sequence.

    q: [B, Lq, Hq, D] raw queries; row r of sequence b is the token at
    absolute position pos0[b] + r.  k_raw, v: [B, Lk, Hkv, D] *unrotated* keys
    and values of positions 0 .. Lk-1 (the prefix followed by the chunk).
    pos0: int or per-sequence list; q_len: None (Lq rows each) or a
    per-sequence count of valid rows (ragged chunks).  Returns O [B, rows,
    heads, D] and LSE [B, heads, rows]; rows r >= q_len[b] give 0 and -inf.

    Row r is row pos0[b] + r of the causal prefill definition: the relation of
    each pair comes from absolute chunk indices, keys sit at j mod s, and keys
    j > pos0[b] + r are masked.  (The DCA guide's "Strategic Recommendations"
    pair DCA with serving that processes long prompts in pieces; a chunk must
    produce exactly the rows the whole prompt would.)
    """
    q = _f64(q)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k_raw.shape[1], k_raw.shape[2]
    s = chunk_size(c, w)
    scale = 1.0 / np.sqrt(D) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    p0 = np.broadcast_to(np.asarray(pos0, dtype=np.int64), (B,))
    ql = np.full(B, Lq, dtype=np.int64) if q_len is None else np.asarray(q_len, dtype=np.int64)
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    O = np.zeros((B, len(rows), len(heads), D))
    LSE = np.full((B, len(heads), len(rows)), -np.inf)
    kpos = key_position(np.arange(Lk), c, w)
    for b in range(B):
        if p0[b] + ql[b] > Lk:
            raise ValueError("the cache must hold every key of the chunk")
        cache = {}
        for hi, h in enumerate(heads):
            g = _kv_head(int(h), Hq, Hkv)
            if g not in cache:
                cache[g] = (rope_rotate(_f64(k_raw[b, :, g]), kpos, base), _f64(v[b, :, g]))
            khat, vg = cache[g]
            for ri, r in enumerate(rows):
                r = int(r)
                if r >= ql[b]:
                    continue
                i = int(p0[b]) + r
                n = i // s
                p_intra, p_succ, p_inter = query_positions(i, c, w)
                S = np.empty(i + 1)
                for lo, hi_, pq in ((n * s, i + 1, p_intra), ((n - 1) * s, n * s, p_succ),
                                    (0, (n - 1) * s, p_inter)):
                    lo = max(lo, 0)
                    if hi_ <= lo:
                        continue
                    S[lo:hi_] = scale * (khat[lo:hi_] @ rope_rotate(q[b, r, h], pq, base))
                o, lse = _softmax_rows(S[None, :], vg[: i + 1])
                O[b, ri, hi] = o[0]
                LSE[b, hi, ri] = lse[0]
    return O, LSE


# ---- paged KV caches ----------------------------------------------------------------
# A serving KV cache ("Dual-Chunk Attention: Training-Free 100k+ Context Guide",
# "Strategic Recommendations": DCA paired with split-KV decoding in serving) is
# often held in fixed-size pages.  The pages describe no page layout; the one
# used here is the common block table: row j of sequence b sits at row j mod P
# of page block_table[b][j // P] of a pool [num_pages, P, H, D].  Paging moves
# rows and changes no arithmetic, so the paged results are the dense ones of
# the gathered sequence.

def paged_rows(pool, block_table, b: int, n: int) -> np.ndarray:
    """Rows 0 .. n-1 of sequence b from a paged pool [num_pages, P, H, D]."""
    pool = np.asarray(pool)
    P = pool.shape[1]
    j = np.arange(n)
    pages = np.asarray(block_table)[b, j // P]
    if np.any(pages < 0) or np.any(pages >= pool.shape[0]):
        raise ValueError("block table entry outside the page pool")
    return pool[pages, j % P]


def dca_decode_paged_ref(q, k_pool_raw, v_pool, block_table, kv_len, c: int, w: int,
                         base: float = 10000.0, sm_scale: float | None = None):
    """Decode against a paged cache of *unrotated* keys: sequence b's cache is
    its first kv_len[b] rows gathered through the block table; its query sits
    at kv_len[b] - 1.  Returns O [B, Hq, D] and LSE [B, Hq]."""
    q = _f64(q)
    B, Hq, D = q.shape
    O = np.zeros((B, Hq, D))
    LSE = np.zeros((B, Hq))
    for b in range(B):
        n = int(kv_len[b])
        kb = _f64(paged_rows(_f64(k_pool_raw), block_table, b, n))[None]
        vb = _f64(paged_rows(_f64(v_pool), block_table, b, n))[None]
        o, lse = dca_decode_ref(q[b: b + 1], kb, vb, c, w, base, sm_scale)
        O[b], LSE[b] = o[0], lse[0]
    return O, LSE


def dca_prefill_chunk_paged_ref(q, k_pool_raw, v_pool, block_table, pos0, c: int, w: int,
                                base: float = 10000.0, sm_scale: float | None = None, q_len=None):
    """Chunked prefill over a paged cache of *unrotated* keys: sequence b's
    keys 0 .. pos0[b] + q_len[b] - 1 are gathered through the block table, then
    the chunk is the dense chunked prefill of that sequence."""
    q = _f64(q)
    B, Lq, Hq, D = q.shape
    p0 = np.broadcast_to(np.asarray(pos0, dtype=np.int64), (B,))
    ql = np.full(B, Lq, dtype=np.int64) if q_len is None else np.asarray(q_len, dtype=np.int64)
    O = np.zeros((B, Lq, Hq, D))
    LSE = np.full((B, Hq, Lq), -np.inf)
    for b in range(B):
        n = int(p0[b] + ql[b])
        kb = _f64(paged_rows(_f64(k_pool_raw), block_table, b, n))[None]
        vb = _f64(paged_rows(_f64(v_pool), block_table, b, n))[None]
        o, lse = dca_prefill_chunk_ref(q[b: b + 1], kb, vb, [int(p0[b])], c, w, base, sm_scale,
                                       q_len=[int(ql[b])])
        O[b], LSE[b] = o[0], lse[0]
    return O, LSE
