/*
 * dca.h - C ABI of the MI355X (gfx950) Dual Chunk Attention library.
 *
 * Dual Chunk Attention (DCA) is the training-free long-context method of
 * "Training-Free Long-Context Scaling of Large Language Models" (abstract),
 * described operationally in "Dual-Chunk Attention: Training-Free 100k+
 * Context Guide" (sections "The Architecture", "Intra-Chunk Attention",
 * "Inter-Chunk Attention", "Successive Chunk Smoothing" and "Flash-DCA").
 *
 * Parameters of every call: pretrain length c, local window w, chunk size
 * s = c - w, RoPE base.  Positions used (0 <= w < c):
 *   key j                          : P_k = j mod s
 *   query i, same chunk (intra)    : P_q = i mod s
 *   query i, previous chunk (succ) : P_q = min(s + (i mod s), c - 1)
 *   query i, older chunks (inter)  : P_q = c - 1
 * The chunk relation of a pair is floor(i/s) - floor(j/s) (0, 1, >= 2).
 * RoPE uses the rotate-half pairing (k, k + D/2) with
 * theta_k = base^(-2k/D); attention is causal with the diagonal included.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises.  Scratch memory comes from the
 *     caller through (ws, ws_bytes); size it with the *_workspace_bytes query.
 *   - Layouts are dense and contiguous: Q/K/V/O are [B, L, H, D] ("BSHD"),
 *     LSE is [B, Hq, L] fp32.  Tensor pointers must be 16-byte aligned and the
 *     workspace 256-byte aligned.
 *   - dtype: DCA_F32 or DCA_BF16, the type of Q/K/V/O (and of caches).  LSE and
 *     all accumulation are fp32.  Head dim D must be 64 or 128.
 *   - GQA: Hq must be a multiple of Hkv; query head h reads KV head
 *     floor(h * Hkv / Hq) (contiguous groups).
 *   - Size limits: B, Hq and Hkv at most 65535 for the prefill entry points
 *     (Hq below 65536 for decode), sequence lengths below 2^30.  The prefill
 *     entry points (whole, SelfExtend, coarse / fine, chunked) also need one
 *     head's key rows, padded to a multiple of 128 rows, below 2^31 bytes:
 *     round_up(L, 128) * D * element size < 2^31, i.e. L <= 2^23 - 128 for
 *     bf16 at D = 128, 2^24 - 128 for bf16 at D = 64 (half of each for fp32);
 *     for the chunked calls L is the largest pos0[b] + q_len[b].  A call
 *     outside these limits returns DCA_ERR_INVALID_ARG (the size queries
 *     return 0).
 *   - stream is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous: a return of DCA_OK means "enqueued".  Device faults surface
 *     at the caller's next synchronisation.
 *   - Argument validation happens before any HIP call, so an invalid call
 *     returns its error without touching the device.  No C++ exception
 *     crosses this interface.  Calls on different streams with distinct
 *     workspaces are independent; the library keeps no global state, except
 *     the static scratch of dca_decode_paged_noalloc (one array per GPU) and
 *     the device address of each GPU's copy of it.
 */
#ifndef DCA_H_
#define DCA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
#define DCA_F32 0
#define DCA_BF16 1

/* Position maps of dca_rope_remap (see the position table above). */
#define DCA_MAP_KEY 0     /* P = t mod s                      */
#define DCA_MAP_Q_INTRA 1 /* P = t mod s                      */
#define DCA_MAP_Q_SUCC 2  /* P = min(s + (t mod s), c - 1)    */
#define DCA_MAP_Q_INTER 3 /* P = c - 1                        */
#define DCA_MAP_PLAIN 4   /* P = t (ordinary RoPE)            */
/* SelfExtend grouped positions (see dca_selfextend_prefill); for these two maps
 * the (c, w) arguments carry the group size G >= 1 and the window W >= 0.     */
#define DCA_MAP_SE_KEY_GROUPED 5 /* P = floor(t / G)                    */
#define DCA_MAP_SE_Q_GROUPED 6   /* P = floor(t / G) + W - floor(W / G) */

/* Status codes. */
#define DCA_OK 0
#define DCA_ERR_INVALID_ARG (-1) /* null pointer, bad shape, w >= c, Hq % Hkv != 0, misalignment,
                                    SelfExtend group < 1 or window < 0                          */
#define DCA_ERR_UNSUPPORTED (-2) /* head dim or dtype the kernels do not implement               */
#define DCA_ERR_WORKSPACE (-3)   /* workspace missing or smaller than the query returned          */
#define DCA_ERR_HIP (-4)         /* a HIP launch reported an error                                */
#define DCA_ERR_TOO_LARGE (-5)   /* dca_decode_paged_noalloc: the call needs more scratch than
                                    DCA_NOALLOC_SCRATCH_BYTES                                    */

/* Bytes of the static device scratch that dca_decode_paged_noalloc uses
 * (one copy per GPU, held until the process ends). */
#define DCA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* Human-readable text for a status code (static storage, never NULL). */
const char* dca_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int dca_version(void);

/*
 * dca_rope_remap - rotate every head vector of x by its DCA position.
 *
 * Definition: the RoPE rotation of "Dual-Chunk Attention: Training-Free 100k+
 * Context Guide", section "The Problem" (angle = position * theta_k per
 * rotary pair), applied at the chunk-local positions of the sections
 * "Intra-Chunk Attention" / "Inter-Chunk Attention" / "Successive Chunk
 * Smoothing" as listed in the header comment.  Token t (0 <= t < L) of x is
 * at absolute position pos0 + t; `map` picks which DCA position it is rotated
 * to.  DCA_MAP_KEY is how a decode KV cache is built; the query maps expose
 * the three query variants the attention kernels form internally.
 *
 *   x, out : [B, L, H, D] of `dtype`, device, 16-byte aligned; out may equal
 *            x (in place).  B, L and H * D are each below 2^31.
 *   pos0   : >= 0, position of token 0.
 *   map    : one of DCA_MAP_*.  For DCA_MAP_SE_KEY_GROUPED / DCA_MAP_SE_Q_GROUPED
 *            c is the SelfExtend group size G (1 <= G <= 2^24) and w the
 *            window W (0 <= W <= 2^30); the DCA rule w < c does not apply.
 * Angles, cos/sin and the rotation are evaluated in fp64; the result is
 * rounded once, to nearest even, into the output type.
 */
int dca_rope_remap(const void* x, void* out, int64_t B, int64_t L, int64_t H, int64_t D,
                   int64_t pos0, int map, int c, int w, double rope_base, int dtype,
                   void* stream);

/*
 * Scratch bytes dca_prefill needs for these sizes (0 on invalid sizes).
 * Holds the query cos/sin table of positions [0, c) (16 bytes reserved per
 * position and frequency: bf16 stores fp32 pairs frequency-major, fp32 fp64
 * pairs), the rotated keys (head-major, padded to a multiple of 128 rows)
 * and the values (bf16: tiled transpose; fp32: a copy).
 */
size_t dca_prefill_workspace_bytes(int64_t B, int64_t L, int64_t Hkv, int64_t D, int c,
                                   int dtype);

/*
 * dca_prefill - DCA causal attention over a whole sequence (prefill).
 *
 * Definition: for every query i and key j <= i, the score is
 *   sm_scale * < R_{P_q(i, rho)} q_i , R_{P_k(j)} k_j >
 * with the query variant chosen by the pair's chunk relation rho ("The
 * Architecture" taxonomy box and the three region sections of the DCA
 * guide); scores are merged with a flash-style online softmax over key tiles
 * ("Flash-DCA: Fusing DCA into FlashAttention Tiling Loops"), so the L x L
 * matrix is never stored.
 *
 *   q         : [B, L, Hq, D] raw (pre-RoPE) queries.
 *   k, v      : [B, L, Hkv, D] raw keys, values.
 *   o         : [B, L, Hq, D] output.
 *   lse       : [B, Hq, L] fp32 natural-log log-sum-exp of the scaled scores,
 *               or NULL.
 *   k_rot_out : [B, L, Hkv, D] keys rotated at j mod s (a decode KV cache), or
 *               NULL.
 *   sm_scale  : softmax scale; <= 0 selects 1/sqrt(D).
 *   ws        : scratch of at least dca_prefill_workspace_bytes(...) bytes.
 * bf16 runs QK^T and PV on bf16 MFMA with fp32 accumulation (rotated q/k and
 * the probabilities are rounded to bf16 before each product; keys are
 * rotated in fp64, queries in fp32 from fp32 angles; the softmax normaliser
 * sums the fp32 probabilities); fp32 runs in fp32 throughout.
 */
int dca_prefill(const void* q, const void* k, const void* v, void* o, float* lse, void* k_rot_out,
                int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int c, int w,
                double rope_base, float sm_scale, int dtype, void* ws, size_t ws_bytes,
                void* stream);

/*
 * The two phases dca_prefill runs, exposed so a caller can prepare K/V once
 * and time or repeat the attention phase on its own.
 *
 * dca_prefill_prepare: builds, inside ws, the query cos/sin table for positions
 * [0, c), the keys rotated at j mod s (head-major, rows padded to a multiple
 * of 128) and the value layout the attention kernel reads (bf16: a tiled
 * transpose; fp32: a copy).  k_rot_out as in dca_prefill (may be NULL).
 *
 * dca_prefill_attend: the fused attention kernel over a workspace prepared by
 * dca_prefill_prepare with the same B, L, Hkv, D, c, w, rope_base and dtype
 * (not checked: a mismatch gives wrong results, not an error).  q, o, lse as
 * in dca_prefill.
 */
int dca_prefill_prepare(const void* k, const void* v, void* k_rot_out, int64_t B, int64_t L,
                        int64_t Hkv, int64_t D, int c, int w, double rope_base, int dtype,
                        void* ws, size_t ws_bytes, void* stream);
int dca_prefill_attend(const void* q, void* o, float* lse, int64_t B, int64_t L, int64_t Hq,
                       int64_t Hkv, int64_t D, int c, int w, float sm_scale, int dtype,
                       const void* ws, size_t ws_bytes, void* stream);

/*
 * The DCA guide's own coarse / fine distances as an alternative position map.
 *
 * Definition: "Dual-Chunk Attention: Training-Free 100k+ Context Guide",
 * sections "Inter-Chunk Attention" and "Successive Chunk Smoothing".  Chunk
 * size C, chunk index c_x = floor(x / C), offset o_x = x mod C, and
 * kappa = target_len / train_len.  For a causal pair (j <= i):
 *   same chunk       : i - j
 *   chunks >= 2 apart: (c_i - c_j) * C / kappa + (o_i - o_j)
 *   adjacent chunks  : (1 - lambda)(i - j) + lambda * (the inter value),
 *                      lambda = o_i / C
 * The distances are real numbers, and the rotation angle of a pair is its
 * distance times theta_k.  They are used as stated, not clamped: the map
 * goes negative when o_j > o_i across several chunks, and can pass
 * train_len past L = target_len.  The kernels factor each distance into a
 * query position minus a key position:
 *   keys at j (same or adjacent chunk) or at c_j C / kappa + o_j (older);
 *   queries at i, i - o_i (1 - 1/kappa) or c_i C / kappa + o_i.
 * These positions and their cos / sin are evaluated in fp64 (for bf16 the
 * query angles are then rounded to fp32).
 *
 * dca_coarse_fine_workspace_bytes: scratch for the fp64 theta table, the
 * (cos, sin) of the three query positions of every row (3 * L * D/2 * 16
 * bytes reserved: fp64 pairs, or fp32 pairs for bf16), the two key rotations
 * and the V layout (0 on invalid sizes).
 * dca_coarse_fine_prefill: q [B, L, Hq, D], k / v [B, L, Hkv, D] raw; o, lse,
 *   sm_scale, GQA, dtypes as in dca_prefill.  chunk >= 1, train_len >= 1,
 *   target_len >= 1.  bf16 needs chunk to be a multiple of 64, so that every
 *   key tile has one relation; otherwise DCA_ERR_UNSUPPORTED.  fp32 takes
 *   any chunk.
 */
size_t dca_coarse_fine_workspace_bytes(int64_t B, int64_t L, int64_t Hkv, int64_t D, int dtype);
int dca_coarse_fine_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                            int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int chunk, int train_len,
                            int target_len, double rope_base, float sm_scale, int dtype, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * dca_prefill_chunk - DCA causal prefill of one chunk of new tokens per
 * sequence, over a KV cache that already holds the sequence's earlier tokens
 * (chunked prefill; ragged batches).
 *
 * Definition: new token r of sequence b is row pos0[b] + r of the dca_prefill
 * definition.  The chunk relation of every pair is taken from absolute
 * positions, so a prompt processed chunk by chunk gives the rows of the whole
 * prompt.  This is the serving side of the DCA guide's "Strategic
 * Recommendations": long prompts are held in a large KV cache.
 *
 *   q        : [B, Lq, Hq, D] raw queries; row r of sequence b is the token at
 *              position pos0[b] + r.
 *   k_cache  : [B, cache_len, Hkv, D] keys rotated at j mod s for positions
 *              0 .. pos0[b] + q_len[b] - 1.  The chunk's own keys must be in
 *              it: write them first with dca_rope_remap(DCA_MAP_KEY, pos0[b]).
 *              Later rows are not read.
 *   v_cache  : [B, cache_len, Hkv, D] values of the same positions.
 *   o        : [B, Lq, Hq, D]; lse : [B, Hq, Lq] fp32 or NULL.  Rows
 *              r >= q_len[b] are left untouched.
 *   pos0     : HOST array of B offsets, pos0[b] >= 0.
 *   q_len    : HOST array of B row counts with 0 <= q_len[b] <= Lq, or NULL
 *              for Lq each.  Also pos0[b] + q_len[b] <= cache_len and
 *              Lq <= cache_len.
 *   ws       : at least dca_prefill_workspace_bytes(B, max_b(pos0[b] + q_len[b]),
 *              Hkv, D, c, dtype) bytes.
 * The host arrays are read during the call only.  The used cache rows are
 * copied into the tiled key / value layout of the workspace, then the prefill
 * kernels run with a query offset per sequence.  The two-group kernel is used
 * when s is a multiple of 64 and every pos0[b] a multiple of 32.  Larger
 * batches are processed in groups of 64 sequences.
 */
int dca_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int64_t* pos0, const int64_t* q_len, int64_t B, int64_t Lq,
                      int64_t cache_len, int64_t Hq, int64_t Hkv, int64_t D, int c, int w,
                      double rope_base, float sm_scale, int dtype, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * SelfExtend-style grouped / neighbor attention through the same prefill
 * kernels.
 *
 * Definition: "LLM Maybe LongLM: Self-Extend LLM Context Window Without
 * Tuning" (abstract) builds two levels of attention from the model's own
 * attention: grouped attention for distant tokens and neighbor attention for
 * tokens within a window.  The abstract states no formula; the positions used
 * are (for causal pairs j <= i, group size G, window W):
 *   i - j <  W (neighbor): query at i, key at j (ordinary RoPE);
 *   i - j >= W (grouped) : query at floor(i/G) + W - floor(W/G), key at
 *                          floor(j/G) -- the grouped distance continues the
 *                          window edge and is never below W.
 * Softmax, scale, LSE, GQA, layouts and dtypes as in dca_prefill.
 *
 * dca_selfextend_workspace_bytes: scratch bytes for these sizes (0 on invalid
 * sizes): the cos/sin table for every position used (fp64; bf16 keeps fp32
 * query pairs there and makes the keys' angles in the kernel), the keys rotated at
 * j and at floor(j/G) (head-major, rows padded to a multiple of 128) and the
 * value layout (bf16: tiled transpose; fp32: a copy).
 *
 * dca_selfextend_prefill:
 *   q      : [B, L, Hq, D] raw queries; k, v : [B, L, Hkv, D] raw keys, values.
 *   o      : [B, L, Hq, D] output; lse : [B, Hq, L] fp32 or NULL.
 *   group  : G >= 1 (G = 1 is ordinary RoPE attention); window : W >= 0
 *            (W >= L is ordinary RoPE attention; W = 0 groups every pair).
 *   ws     : scratch of at least dca_selfextend_workspace_bytes(...) bytes.
 * Key tiles holding grouped pairs and those holding neighbor pairs are visited
 * in turn; tiles on the window edge twice, each time with the other class
 * masked, merged by the online softmax.
 */
size_t dca_selfextend_workspace_bytes(int64_t B, int64_t L, int64_t Hkv, int64_t D, int group,
                                      int window, int dtype);
int dca_selfextend_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int group,
                           int window, double rope_base, float sm_scale, int dtype, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Scratch bytes dca_decode needs for these sizes (0 on invalid sizes): the
 * three rotated query variants and the per-split partial results.
 */
size_t dca_decode_workspace_bytes(int64_t B, int64_t kv_len, int64_t Hq, int64_t Hkv, int64_t D,
                                  int dtype);

/*
 * dca_decode - one new query token per sequence against a long KV cache.
 *
 * Definition: row q_pos = kv_len - 1 of dca_prefill (the cache holds the new
 * token itself), computed split-K: the cache is cut into key ranges processed
 * in parallel and merged by log-sum-exp ("Strategic Recommendations": pair
 * DCA with FlashDecoding, which splits the KV cache across the GPU).
 *
 *   q        : [B, Hq, D] raw query of the new token.
 *   k_cache  : [B, kv_len, Hkv, D] keys ALREADY rotated at j mod s (from
 *              dca_rope_remap(DCA_MAP_KEY, pos0 = 0) or dca_prefill's k_rot_out).
 *   v_cache  : [B, kv_len, Hkv, D] values.
 *   o        : [B, Hq, D] output; lse : [B, Hq] fp32 or NULL.
 *   ws       : scratch of at least dca_decode_workspace_bytes(...) bytes.
 */
int dca_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
               int64_t B, int64_t kv_len, int64_t Hq, int64_t Hkv, int64_t D, int c, int w,
               double rope_base, float sm_scale, int dtype, void* ws, size_t ws_bytes,
               void* stream);

/*
 * dca_decode_varlen - dca_decode for a ragged batch: sequence b holds kv_len[b]
 * cached tokens (its new token included) and its new token sits at position
 * kv_len[b] - 1.
 *
 *   kv_len   : HOST array of B lengths, 1 <= kv_len[b] <= cache_len (read
 *              during the call only).
 *   k_cache, v_cache : [B, cache_len, Hkv, D]; rows >= kv_len[b] are not read.
 *   ws       : at least dca_decode_varlen_workspace_bytes(kv_len, B, Hq, Hkv, D,
 *              dtype) bytes (0 there on invalid sizes).
 * Everything else as in dca_decode.  The key-range length spreads the whole
 * batch's keys over one round of waves; ranges past a sequence's end
 * contribute nothing to the merge.  Larger batches are processed in groups
 * of 64 sequences.
 */
size_t dca_decode_varlen_workspace_bytes(const int64_t* kv_len, int64_t B, int64_t Hq, int64_t Hkv,
                                         int64_t D, int dtype);
int dca_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int64_t* kv_len, int64_t B, int64_t cache_len, int64_t Hq, int64_t Hkv,
                      int64_t D, int c, int w, double rope_base, float sm_scale, int dtype, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * Paged KV caches: dca_decode_paged and dca_prefill_chunk_paged.
 *
 * Definition: the same results as dca_decode_varlen and dca_prefill_chunk
 * for the sequence whose cached row j is row j mod page_size of page
 * block_table[b][j / page_size].  Paging moves rows only.  The pages describe
 * no page layout; this block table is the common one of serving KV caches
 * (the DCA guide's "Strategic Recommendations" pair DCA with split-KV
 * decoding for serving long contexts).
 *
 *   k_pages, v_pages : page pools [num_pages, page_size, Hkv, D] (keys rotated
 *              at j mod s, as for the dense caches).
 *   block_table : DEVICE array int32 [B, max_blocks]: the page of each block of
 *              page_size rows of each sequence.  Entries past a sequence's last
 *              used block are not read.  An entry outside [0, num_pages) is
 *              never dereferenced; the results of that sequence that would
 *              use it become NaN (others of the same sequence may too).
 *   page_size : a multiple of 16 (so every 16-row half of the decode kernel's
 *              32-key sub-tiles lies inside one page).
 *   kv_len / pos0 + q_len : at most max_blocks * page_size.
 *   ws       : decode: dca_decode_varlen_workspace_bytes(kv_len, ...); chunk:
 *              dca_prefill_workspace_bytes(B, max_b(pos0[b] + q_len[b]), ...).
 * Everything else as in dca_decode_varlen / dca_prefill_chunk.  Pool rows that
 * no table entry names are never read.
 */
int dca_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                     void* o, float* lse, const int64_t* kv_len, int64_t B, int64_t num_pages,
                     int64_t page_size, int64_t max_blocks, int64_t Hq, int64_t Hkv, int64_t D, int c,
                     int w, double rope_base, float sm_scale, int dtype, void* ws, size_t ws_bytes,
                     void* stream);
int dca_prefill_chunk_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int32_t* block_table, void* o, float* lse, const int64_t* pos0,
                            const int64_t* q_len, int64_t B, int64_t Lq, int64_t num_pages,
                            int64_t page_size, int64_t max_blocks, int64_t Hq, int64_t Hkv, int64_t D,
                            int c, int w, double rope_base, float sm_scale, int dtype, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * dca_decode_paged_noalloc - dca_decode_paged without a workspace argument,
 * for callers that cannot allocate device memory: code recorded into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments (minus ws / ws_bytes), same kernels and bit-identical
 * results as dca_decode_paged.  The scratch the decode needs (rotated query
 * variants and the per-key-range partial O / LSE, the size
 * dca_decode_varlen_workspace_bytes(kv_len, B, Hq, Hkv, D, dtype) reports)
 * comes from a static device array of DCA_NOALLOC_SCRATCH_BYTES (32 MiB) in
 * the library; a call needing more returns DCA_ERR_TOO_LARGE before touching
 * the device (e.g. B * Hq * (key ranges) * D * 4 bytes of partials: the
 * 16 x 64-head, 100k-token decode needs about 9 MiB).  The call allocates
 * nothing (no hipMalloc / hipFree, no host-side allocation for DCA); the
 * first call on a device looks up that device's copy of the array with
 * hipGetSymbolAddress.  The array is shared by every call on the same GPU
 * and keeps the last call's contents (nothing in it needs to start at zero):
 * calls that overlap on one GPU (on different streams, or from several host
 * threads) race on it and must be serialised by the caller.  The current
 * device must be the one that holds the tensors.
 */
int dca_decode_paged_noalloc(const void* q, const void* k_pages, const void* v_pages,
                             const int32_t* block_table, void* o, float* lse, const int64_t* kv_len,
                             int64_t B, int64_t num_pages, int64_t page_size, int64_t max_blocks,
                             int64_t Hq, int64_t Hkv, int64_t D, int c, int w, double rope_base,
                             float sm_scale, int dtype, void* stream);

/*
 * Decode under the SelfExtend and coarse / fine maps.
 *
 * Definition: the new token of sequence b is row kv_len[b] - 1 of
 * dca_selfextend_prefill (resp. dca_coarse_fine_prefill) over its first
 * kv_len[b] cached tokens ("LLM Maybe LongLM: Self-Extend LLM Context Window
 * Without Tuning", abstract; "Dual-Chunk Attention: Training-Free 100k+
 * Context Guide", sections "Inter-Chunk Attention" and "Successive Chunk
 * Smoothing"), computed split-K like dca_decode_varlen.  Both maps give a key
 * one of two rotations, so the caller keeps two rotated key caches:
 *   SelfExtend:    k_cache at j (dca_rope_remap DCA_MAP_PLAIN) for the
 *                  neighbor keys j > q_pos - W, k_cache_grouped at floor(j/G)
 *                  (DCA_MAP_SE_KEY_GROUPED, c = G, w = W) for the others;
 *   coarse / fine: k_cache at j (DCA_MAP_PLAIN) for keys in the new token's
 *                  chunk and the one before, k_cache_scaled at
 *                  floor(j/C) C/kappa + j mod C (dca_coarse_fine_key_remap)
 *                  for older keys.
 * Each key is read from one of the two caches only.  q [B, Hq, D] raw;
 * caches and v_cache [B, cache_len, Hkv, D]; kv_len HOST array (1 <=
 * kv_len[b] <= cache_len); o, lse, sm_scale, GQA, dtypes and errors as in
 * dca_decode_varlen.  The workspace queries return 0 on invalid sizes.
 *
 * dca_coarse_fine_key_remap: x [B, L, H, D] at positions pos0 .. pos0 + L - 1
 * rotated at the coarse-scaled key positions (fp64 angles, one rounding),
 * written to out (may alias x only if identical); 16-byte aligned, with B,
 * L and H * D each below 2^31.
 */
size_t dca_selfextend_decode_workspace_bytes(const int64_t* kv_len, int64_t B, int64_t Hq, int64_t Hkv,
                                             int64_t D, int group, int window, int dtype);
int dca_selfextend_decode(const void* q, const void* k_cache, const void* k_cache_grouped, const void* v_cache,
                          void* o, float* lse, const int64_t* kv_len, int64_t B, int64_t cache_len,
                          int64_t Hq, int64_t Hkv, int64_t D, int group, int window, double rope_base,
                          float sm_scale, int dtype, void* ws, size_t ws_bytes, void* stream);
size_t dca_coarse_fine_decode_workspace_bytes(const int64_t* kv_len, int64_t B, int64_t Hq, int64_t Hkv,
                                              int64_t D, int chunk, int dtype);
int dca_coarse_fine_decode(const void* q, const void* k_cache, const void* k_cache_scaled, const void* v_cache,
                           void* o, float* lse, const int64_t* kv_len, int64_t B, int64_t cache_len,
                           int64_t Hq, int64_t Hkv, int64_t D, int chunk, int train_len, int target_len,
                           double rope_base, float sm_scale, int dtype, void* ws, size_t ws_bytes,
                           void* stream);
int dca_coarse_fine_key_remap(const void* x, void* out, int64_t B, int64_t L, int64_t H, int64_t D,
                              int64_t pos0, int chunk, int train_len, int target_len, double rope_base,
                              int dtype, void* stream);

/*
 * dca_selfextend_decode_paged, dca_coarse_fine_decode_paged: the two map
 * decodes above over page pools, with the same results (paging moves rows
 * only; see dca_decode_paged for the block-table layout and its rules).
 *
 *   k_pages, k_pages_2nd, v_pages : pools [num_pages, page_size, Hkv, D]; the
 *              two key pools hold the two rotations of the same rows
 *              (k_pages at j; k_pages_2nd grouped, resp. coarse-scaled), so
 *              one block table addresses all three pools.
 *   block_table : DEVICE int32 [B, max_blocks]; page_size a multiple of 16;
 *              kv_len[b] <= max_blocks * page_size.
 *   ws       : dca_selfextend_decode_workspace_bytes, resp.
 *              dca_coarse_fine_decode_workspace_bytes (as for the dense caches).
 * An entry outside [0, num_pages) is never dereferenced; results of that
 * sequence that would use it become NaN.  Everything else as in the dense
 * map decodes.
 */
int dca_selfextend_decode_paged(const void* q, const void* k_pages, const void* k_pages_2nd, const void* v_pages,
                                const int32_t* block_table, void* o, float* lse, const int64_t* kv_len, int64_t B,
                                int64_t num_pages, int64_t page_size, int64_t max_blocks, int64_t Hq, int64_t Hkv,
                                int64_t D, int group, int window, double rope_base, float sm_scale, int dtype,
                                void* ws, size_t ws_bytes, void* stream);
int dca_coarse_fine_decode_paged(const void* q, const void* k_pages, const void* k_pages_2nd, const void* v_pages,
                                 const int32_t* block_table, void* o, float* lse, const int64_t* kv_len, int64_t B,
                                 int64_t num_pages, int64_t page_size, int64_t max_blocks, int64_t Hq, int64_t Hkv,
                                 int64_t D, int chunk, int train_len, int target_len, double rope_base,
                                 float sm_scale, int dtype, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCA_H_ */
