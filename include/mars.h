/*
 * mars.h — C ABI of the MARS hot-path library (libmars.so, gfx950 / MI355X).
 *
 * MARS ("MARS: Enabling Autoregressive Models Multi-Token Generation", Jin,
 * Wang, Luo, Sun) trains an unchanged autoregressive transformer on a
 * two-stream input z = [x; x~] under a structured 2L x 2L attention mask, and
 * at inference appends B [MASK] queries per sequence, scores them with the
 * ordinary LM head and accepts a left-to-right prefix whose max-probability
 * stays at or above a threshold tau. This library holds the data-parallel hot
 * path of that method:
 *
 *   mars_attn_two_stream    two-stream masked attention forward (training form)
 *   mars_attn_two_stream_bwd  its dq, dk, dv (training)
 *   mars_attn_causal        causal attention over any length (no-cache prefill)
 *   mars_attn_block_decode  B mask queries against a paged block-level KV cache
 *   mars_attn_block_decode_rows  the same with a per-sequence row count
 *   mars_lmhead_confidence  LM-head GEMM + per-position argmax / max-softmax
 *   mars_lmhead_confidence_packed  the same on weights packed by mars_lmhead_pack
 *   mars_lmhead_confidence_noalloc the same with no workspace argument
 *   mars_accept_commit      left-to-right acceptance + KV commit of the prefix
 *   mars_accept_commit_layers  the same, committing into every layer's cache
 *   mars_kv_append          paged KV append of a prompt
 *   mars_block_sync_accept  acceptance under the batch-synchronous block cache
 *   mars_block_freeze       freezes a full block into the paged cache
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller. The library
 *    allocates no device memory and keeps no state between calls; scratch
 *    space, where needed, is a caller-provided `workspace` whose size the
 *    matching *_workspace_bytes() helper returns (mars_lmhead_confidence_noalloc
 *    alone uses a fixed library-owned array instead; see there).
 *  - Tensors are dense, row-major (C order), in the layouts stated per call.
 *    Every tensor pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work: they never synchronise the host, never print and
 *    never allocate. Results are deterministic run to run (no atomics whose
 *    order could change a value).
 *  - Return value: MARS_OK (0) or a negative MARS_ERR_* code, checked on the
 *    host before anything is enqueued (argument errors) or right after the
 *    launch (MARS_ERR_LAUNCH). A non-zero return means nothing was written.
 *  - Errors that only the device can see (a cache position beyond the pages a
 *    sequence owns, a block-table entry outside [0, num_pages), a non-finite
 *    logit) are OR-ed as bit flags into an optional caller-owned int32
 *    `status` word (pass NULL to ignore them). Kernels never read or write out
 *    of bounds because of such input: the affected keys are dropped, the
 *    affected rows are not written, and the flag is raised.
 *  - softmax_scale <= 0 selects 1/sqrt(head_dim).
 */
#ifndef MARS_H_
#define MARS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes */
#define MARS_OK               0
#define MARS_ERR_NULL        -1  /* a required pointer is NULL                         */
#define MARS_ERR_SHAPE       -2  /* a size is out of range or sizes disagree           */
#define MARS_ERR_DTYPE       -3  /* unknown dtype code                                 */
#define MARS_ERR_UNSUPPORTED -4  /* valid but not built (e.g. this head_dim)           */
#define MARS_ERR_ALIGN       -5  /* a tensor pointer is not 16-byte aligned            */
#define MARS_ERR_WORKSPACE   -6  /* workspace NULL or smaller than required            */
#define MARS_ERR_LAUNCH      -7  /* the HIP runtime reported an error at launch        */

/* dtype codes (element type of Q/K/V/O and of the KV cache) */
#define MARS_F32  0
#define MARS_BF16 1

/* Device status bit flags (sticky; OR-ed into *status) */
#define MARS_STATUS_CACHE_OVERFLOW 1  /* a position reached max_pages * page_size     */
#define MARS_STATUS_BAD_PAGE       2  /* a block_table entry outside [0, num_pages)   */
#define MARS_STATUS_NONFINITE      4  /* a logit row held NaN or +-Inf                */

/*
 * Two-stream MARS attention forward (training form).
 *
 * Defines: the 2L x 2L mask M over z = [x; x~] of the papernotes.org notes,
 * key design 1 (关键设计 1), equation M_ij, with block index
 * beta(t) = ceil(t / B) on 1-based t: clean rows attend causally to the clean
 * stream; a mask row attends causally inside its own block of the mask stream
 * and to the clean tokens of strictly earlier blocks. One forward pass over z,
 * as in the notes' overall framework (整体框架).
 * In 0-based form, for query a and key c in [0, 2L), t = a - L, b = t / B:
 *   a <  L : visible iff c <= a
 *   a >= L : visible iff c < b*B  or  L + b*B <= c <= a
 * mask_mode = 1 replaces M by plain causal attention over all 2L positions
 * (the dense comparison the mask is measured against).
 *
 * q   [batch, 2L, n_q_heads,  head_dim]   dtype
 * k,v [batch, 2L, n_kv_heads, head_dim]   dtype
 * o   [batch, 2L, n_q_heads,  head_dim]   dtype (written)
 * lse [batch, n_q_heads, 2L] float32, natural-log sum-exp of the scaled,
 *     masked scores per row (written); may be NULL.
 * Query head h reads KV head h / (n_q_heads / n_kv_heads).
 * Supported: dtype MARS_BF16 with head_dim 64 or 128 (MFMA path);
 *            dtype MARS_F32  with head_dim 32, 64 or 128.
 * The fp32 path is a full-precision check path, not a fast one: one lane per
 * query row holds its q and o rows in registers (head_dim 128: 256 VGPRs + 135
 * accumulation registers, one wave per SIMD; 64: 213 VGPRs; 32: 117) and K/V
 * pass through LDS 32 keys at a time with scalar FMAs.
 * Limits: 1 <= B <= L, 2L <= 2^30, n_q_heads % n_kv_heads == 0.
 */
int mars_attn_two_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                         int32_t batch, int32_t L, int32_t B, int32_t n_q_heads,
                         int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                         float softmax_scale, int32_t mask_mode, void* stream);

/*
 * Causal attention over T positions: the no-cache prefill, in which every step
 * recomputes the whole sequence (prompt plus the B [MASK] rows) causally
 * (gist.science explainer, section 4; papernotes.org notes, wall-clock table,
 * no-cache row).
 *
 * q [batch, T, n_q_heads, head_dim], k/v [batch, T, n_kv_heads, head_dim],
 * o as q; lse optional [batch, n_q_heads, T]. T may be odd. Same dtypes, head
 * sizes, scale default, errors and determinism as mars_attn_two_stream in its
 * causal mode (which this is, with the two-stream split removed).
 */
int mars_attn_causal(const void* q, const void* k, const void* v, void* o, float* lse,
                     int32_t batch, int32_t T, int32_t n_q_heads, int32_t n_kv_heads,
                     int32_t head_dim, int32_t dtype, float softmax_scale, void* stream);

/*
 * Append T rows per sequence to the paged KV cache (fills the block-level
 * cache from a prefill; notes, key design 4 (关键设计 4)). Row r of sequence s
 * goes to position cache_len[s] + r, in the layouts of mars_attn_block_decode
 * (K [pages, Hkv, page, d], V [pages, Hkv, d, page]); then cache_len[s]
 * advances by the rows that fit in the sequence's max_pages * page_size
 * capacity.
 *
 * k_rows, v_rows [S, T, n_kv_heads, head_dim] (dtype MARS_BF16 or MARS_F32;
 * head_dim a multiple of 8 with head_dim * element size <= 512 bytes, else
 * MARS_ERR_UNSUPPORTED; S <= 65535, n_kv_heads <= 65535);
 * block_table [S, max_pages] int32; cache_len [S] int32 (updated in place).
 * Rows past the capacity or on a page id outside [0, num_pages) are skipped
 * and raise MARS_STATUS_CACHE_OVERFLOW / MARS_STATUS_BAD_PAGE in `status`
 * (optional). Two launches on `stream`: the copy, then the length update.
 */
int mars_kv_append(const void* k_rows, const void* v_rows, void* k_cache, void* v_cache,
                   const int32_t* block_table, int32_t* cache_len, int32_t S, int32_t T,
                   int32_t n_kv_heads, int32_t head_dim, int32_t page_size, int32_t max_pages,
                   int32_t num_pages, int32_t dtype, int32_t* status, void* stream);

/*
 * Acceptance under the batch-synchronous block cache (papernotes.org notes,
 * key design 4 (关键设计 4): the prefix cache grows by whole blocks of B_cache
 * tokens once every sequence of the batch has filled the block; the batch
 * advances by the smallest accepted count, faster sequences waiting at the
 * block boundary).
 *
 * p_max, top_id [S, B] and tau [S] as for mars_accept_commit (the accepted
 * count n_s is the same leading-run rule). State, device memory owned by the
 * caller and updated in place: unfrozen [S] int32, tokens accepted since the
 * last frozen block (0 .. B_cache; start at 0); block_tokens [S, B_cache]
 * int32, their ids (-1 past unfrozen[s]). One step:
 *   1. if unfrozen[s] == B_cache for every s, the forward of this step froze
 *      the block (see mars_block_freeze): unfrozen restarts at 0 and
 *      block_tokens at -1;
 *   2. policy 0 (batch minimum): every sequence keeps min over s of n_s,
 *      capped at B_cache - unfrozen[s]; policy 1 (wait at the boundary):
 *      sequence s keeps n_s, capped the same way;
 *   3. the kept top ids are written to block_tokens[s, unfrozen[s] ...] and
 *      unfrozen[s] grows by the kept count.
 * Outputs: n_kept [S] int32 (the kept count), n_rows [S] int32 =
 * unfrozen[s] + B, the new-row count of the next forward (for
 * mars_attn_block_decode_rows). One workgroup for the whole batch.
 * status optional: MARS_STATUS_CACHE_OVERFLOW if an unfrozen count was outside
 * [0, B_cache] (it is clamped). Limits: S <= 2^24, B <= 64, B_cache <= 4096.
 */
int mars_block_sync_accept(const float* p_max, const int32_t* top_id, const float* tau,
                           int32_t* unfrozen, int32_t* block_tokens, int32_t* n_kept,
                           int32_t* n_rows, int32_t S, int32_t B, int32_t B_cache,
                           int32_t policy, int32_t* status, void* stream);

/*
 * Freeze the block into the paged cache: if unfrozen[s] == B_cache for every
 * s (checked on the device), the first B_cache rows of k_rows / v_rows
 * [S, R, n_kv_heads, head_dim] (the K/V of the forward whose first rows are
 * the block's tokens) are appended at cache_len[s] as by mars_kv_append, and
 * cache_len[s] grows by B_cache; otherwise nothing is written (notes, key
 * design 4 (关键设计 4): the cache is frozen by one forward at the block
 * crossing). Run it after that forward's attention and before
 * mars_block_sync_accept of the same step, on the same stream. Same dtypes,
 * layouts, limits and status flags as mars_kv_append; B_cache <= R.
 */
int mars_block_freeze(const void* k_rows, const void* v_rows, void* k_cache, void* v_cache,
                      const int32_t* block_table, int32_t* cache_len, const int32_t* unfrozen,
                      int32_t S, int32_t R, int32_t B_cache, int32_t n_kv_heads,
                      int32_t head_dim, int32_t page_size, int32_t max_pages, int32_t num_pages,
                      int32_t dtype, int32_t* status, void* stream);

/*
 * Two-stream MARS attention backward: dq, dk, dv of mars_attn_two_stream.
 *
 * Defines: the pages train the unchanged model on L_mask + L_AR through the
 * two-stream attention (papernotes.org notes, key design 2 (关键设计 2);
 * gist.science explainer, section 2B), so a training step needs the gradient
 * of that attention. With S = scale Q K^T under the mask of key design 1,
 * P = softmax(S), O = P V: dV = P^T dO, dS = P * (dO V^T - rowsum(dO * O)),
 * dQ = scale dS K, dK = scale dS^T Q; a KV head sums over its query heads.
 *
 * q, d_o, o, dq [batch, 2L, n_q_heads, head_dim]; k, v, dk, dv
 * [batch, 2L, n_kv_heads, head_dim]; all bf16 (dtype MARS_BF16), head_dim 64
 * or 128. o and lse [batch, n_q_heads, 2L] (float32, natural log) are the
 * forward's outputs for the same q, k, v, B, scale and mask_mode. dq, dk, dv
 * are written (every element); the inputs are not modified.
 * workspace >= mars_attn_two_stream_bwd_workspace_bytes(batch, L, n_q_heads,
 * n_kv_heads, head_dim) bytes of device memory.
 * Errors: as mars_attn_two_stream; MARS_ERR_DTYPE for fp32; MARS_ERR_UNSUPPORTED
 * for other head sizes; MARS_ERR_WORKSPACE if the workspace is missing or
 * small. Deterministic: no atomics, so repeated calls on one GPU give the same
 * bits. (How many query heads one dK/dV workgroup sums in registers follows
 * the GPU's compute-unit count, so the summation order of dk, dv can differ
 * between GPUs of different sizes.)
 */
int mars_attn_two_stream_bwd(const void* q, const void* k, const void* v, const void* o,
                             const void* d_o, const float* lse, void* dq, void* dk, void* dv,
                             int32_t batch, int32_t L, int32_t B, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                             float softmax_scale, int32_t mask_mode, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Workspace bytes mars_attn_two_stream_bwd needs (0 on bad sizes): the rowsum
 * per (batch, query head, row), plus room for fp32 dK/dV partials of every query
 * head when n_q_heads > n_kv_heads (one partial per set of consecutive query
 * heads that a workgroup serves; they are summed per KV head in head order). */
size_t mars_attn_two_stream_bwd_workspace_bytes(int32_t batch, int32_t L, int32_t n_q_heads,
                                                int32_t n_kv_heads, int32_t head_dim);

/*
 * Block-decode attention (inference form).
 *
 * Defines: each sequence appends B [MASK] queries; a single forward scores all
 * B positions (gist.science explainer, section 2C; papernotes.org notes, key
 * design 3), with the B mask queries reading the block-level prefix KV cache
 * (notes, key design 4 (关键设计 4); explainer, section 2D). Row r of sequence
 * s attends to cache positions 0 .. cache_len[s]-1 and, causally, to the new
 * rows 0 .. r of the same step.
 *
 * q        [S, B, n_q_heads,  head_dim]  bf16
 * k_new    [S, B, n_kv_heads, head_dim]  bf16  (K of the B new rows)
 * v_new    [S, B, n_kv_heads, head_dim]  bf16
 * k_cache  [num_pages, n_kv_heads, page_size, head_dim]  bf16
 * v_cache  [num_pages, n_kv_heads, head_dim, page_size]  bf16 (V is stored
 *          transposed inside each page)
 * block_table [S, max_pages] int32: cache position p of sequence s lives in
 *          page block_table[s, p / page_size], slot p % page_size.
 * cache_len   [S] int32 (device): cached prefix length per sequence.
 * o        [S, B, n_q_heads, head_dim]  bf16 (written)
 * workspace: >= mars_decode_workspace_bytes(...) bytes of device memory
 *          (split-K partial results; contents on entry are ignored).
 * status   optional: MARS_STATUS_CACHE_OVERFLOW if cache_len[s] exceeds
 *          max_pages * page_size (the excess is ignored), MARS_STATUS_BAD_PAGE
 *          for a table entry outside [0, num_pages) (its keys are dropped).
 * Supported: dtype MARS_BF16, head_dim 64 or 128, page_size a multiple of 16,
 *          1 <= B <= 64, n_q_heads <= 4096.
 */
int mars_attn_block_decode(const void* q, const void* k_new, const void* v_new,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* cache_len, void* o,
                           int32_t S, int32_t B, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, int32_t page_size, int32_t max_pages,
                           int32_t num_pages, int32_t dtype, float softmax_scale,
                           void* workspace, size_t workspace_bytes, int32_t* status,
                           void* stream);

/*
 * Block-decode attention with a per-sequence number of new rows: the forward
 * of the batch-synchronous block cache (notes, key design 4 (关键设计 4)),
 * whose new rows for sequence s are the u_s tokens accepted since the last
 * frozen block followed by the B [MASK] rows.
 *
 * As mars_attn_block_decode with B replaced by R, the row capacity of q,
 * k_new, v_new and o ([S, R, ...]), plus n_rows [S] int32 (device): sequence s
 * uses its first min(max(n_rows[s], 0), R) rows; row r of them attends to the
 * cache prefix and to new rows 0 .. r. Output rows past n_rows[s] are not
 * written. Workspace: mars_decode_workspace_bytes(S, R, ...).
 */
int mars_attn_block_decode_rows(const void* q, const void* k_new, const void* v_new,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* cache_len,
                                const int32_t* n_rows, void* o, int32_t S, int32_t R,
                                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                int32_t page_size, int32_t max_pages, int32_t num_pages,
                                int32_t dtype, float softmax_scale, void* workspace,
                                size_t workspace_bytes, int32_t* status, void* stream);

/* Workspace bytes mars_attn_block_decode needs for these sizes (0 on bad sizes). */
size_t mars_decode_workspace_bytes(int32_t S, int32_t B, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int32_t page_size, int32_t max_pages);

/*
 * LM-head GEMM + confidence.
 *
 * Defines: the unchanged LM head produces logits for all B positions in one
 * forward (gist.science explainer, sections 2C and 3); the confidence of a
 * position is max_v p(x_t = v) under the softmax of its logits (papernotes.org
 * notes, key design 3 (关键设计 3)). Per row: m = max_v l_v, top_id = the
 * smallest v with l_v = m, p_max = 1 / sum_v exp(l_v - m).
 *
 * hidden  [N, D] bf16, or NULL: then `logits` is an INPUT and only the
 *         confidence step runs.
 * w_lm    [V, D] bf16 (one row per vocabulary entry); ignored if hidden NULL.
 * logits  [N, V] float32: written (= hidden . w_lm^T, fp32 accumulation) when
 *         hidden != NULL, read otherwise. May be NULL when hidden != NULL:
 *         then the confidence is reduced inside the GEMM (per row and
 *         vocabulary tile of 320 entries, or 64 in a tail launch: max, lowest
 *         argmax, sum of exp) and no logits are written. top_id is identical to the unfused call (same
 *         fp32 values); p_max agrees to fp32 rounding of the sum order.
 * top_id  [N] int32, p_max [N] float32 (written).
 * workspace >= mars_lmhead_workspace_bytes(N, V) bytes (covers both forms).
 * status  optional: MARS_STATUS_NONFINITE if a row held NaN/Inf (that row's
 *         p_max is then NaN or 0). The fused form detects NaN and +Inf.
 * Limits: D % 32 == 0 when hidden != NULL; V % 4 == 0; 1 <= N <= 65535.
 */
int mars_lmhead_confidence(const void* hidden, const void* w_lm, float* logits, int32_t N,
                           int32_t D, int32_t V, int32_t* top_id, float* p_max,
                           void* workspace, size_t workspace_bytes, int32_t* status,
                           void* stream);

/* Workspace bytes mars_lmhead_confidence needs (0 on bad sizes). */
size_t mars_lmhead_workspace_bytes(int32_t N, int32_t V);

/*
 * Weight packing for the LM-head GEMM (done once, when the weights are
 * loaded). A row-major W [V, D] makes each 32-wide K stage of the GEMM read 64
 * bytes from each of 320 rows 2D bytes apart; the packed layout
 * [ceil(V / 320)][D / 32][320][32] bf16 (rows past V are zeros) makes every
 * stage one contiguous 20 KiB block. The products, and so the logits, ids and
 * probabilities, are bit-identical to the row-major call.
 *
 * mars_lmhead_packed_bytes: size of the packed buffer (0 unless D >= 32,
 * D % 32 == 0, V >= 4 and V % 4 == 0). mars_lmhead_pack: w_lm [V, D] bf16 ->
 * w_packed (that many bytes, 16-byte aligned), enqueued on `stream`.
 * mars_lmhead_confidence_packed: as mars_lmhead_confidence with an LM head
 * (hidden and w_packed required, logits NULL for the fused form).
 */
size_t mars_lmhead_packed_bytes(int32_t D, int32_t V);
int mars_lmhead_pack(const void* w_lm, void* w_packed, int32_t D, int32_t V, void* stream);
int mars_lmhead_confidence_packed(const void* hidden, const void* w_packed, float* logits,
                                  int32_t N, int32_t D, int32_t V, int32_t* top_id,
                                  float* p_max, void* workspace, size_t workspace_bytes,
                                  int32_t* status, void* stream);

/*
 * mars_lmhead_confidence without a workspace argument: the entry point for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * Arguments, layouts, results and errors as mars_lmhead_confidence (row-major
 * w_lm; hidden may be NULL for the confidence alone). The confidence partials
 * live in a library-owned device array of MARS_NOALLOC_SCRATCH_BYTES per GPU,
 * created with the library's code object on each GPU and held until the
 * process ends; the call allocates nothing. It needs N * P * 16 bytes of that
 * array, where P is the number of vocabulary tiles of the GEMM (about V / 320)
 * when the confidence is fused into the LM head (hidden != NULL, logits ==
 * NULL), else the number of row chunks of the confidence pass (at most 32);
 * beyond MARS_NOALLOC_SCRATCH_BYTES it returns MARS_ERR_WORKSPACE and enqueues
 * nothing. At V = 152064 the fused form takes up to 2202 rows.
 * Every call on one GPU shares that GPU's array and leaves its partials there:
 * calls that may overlap on one GPU (other streams, no ordering between them)
 * race on it and must not be made. No part of the array needs to start at
 * zero (each partial is written before it is read).
 */
#define MARS_NOALLOC_SCRATCH_BYTES (16u << 20)
int mars_lmhead_confidence_noalloc(const void* hidden, const void* w_lm, float* logits,
                                   int32_t N, int32_t D, int32_t V, int32_t* top_id,
                                   float* p_max, int32_t* status, void* stream);

/*
 * Left-to-right acceptance + KV commit of the accepted prefix.
 *
 * Defines: tokens are accepted from left to right while p_max >= tau, up to
 * the first position below tau, and at least the first token is always
 * accepted (papernotes.org notes, key design 3 (关键设计 3); gist.science
 * explainer, section 2C; tau = 1 gives one token per step). tau is per
 * sequence and may change between calls (explainer, sections 2C and 5). The
 * accepted tokens join the persistent prefix cache (notes, key design 4).
 * Per sequence s:
 *   n = max(1, length of the leading run of p_max[s, r] >= tau[s])
 *   accepted_ids[s, r] = top_id[s, r] for r < n, else -1
 *   rows r < n of k_new/v_new go to cache positions cache_len[s] + r
 *   commit_pos[s, r] = that position, or -1; cache_len[s] += rows written.
 *
 * p_max [S, B] float32, top_id [S, B] int32, tau [S] float32 (device).
 * k_new, v_new [S, B, n_kv_heads, head_dim] dtype; caches as in
 * mars_attn_block_decode (K [pages, Hkv, page, d], V [pages, Hkv, d, page]).
 * cache_len [S] int32, read and updated in place.
 * n_accepted [S], accepted_ids [S, B], commit_pos [S, B] int32 (written).
 * status optional: a row that would pass max_pages * page_size is not written
 * (MARS_STATUS_CACHE_OVERFLOW); a row whose page id is outside [0, num_pages)
 * is not written (MARS_STATUS_BAD_PAGE); cache_len then advances only by the
 * rows written before the first such row.
 * NaN p_max compares false (the scan stops there).
 * Limits: 1 <= B <= 64; dtype MARS_BF16 or MARS_F32; head_dim % 8 == 0.
 */
int mars_accept_commit(const float* p_max, const int32_t* top_id, const float* tau,
                       const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       const int32_t* block_table, int32_t* cache_len, int32_t* n_accepted,
                       int32_t* accepted_ids, int32_t* commit_pos, int32_t S, int32_t B,
                       int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                       int32_t max_pages, int32_t num_pages, int32_t dtype, int32_t* status,
                       void* stream);

/*
 * The same acceptance, then the commit into every layer's cache at once (the
 * accepted tokens join each layer's prefix cache: notes, key design 4
 * (关键设计 4); a model keeps one KV cache per decoder layer).
 *
 * The decision, n_accepted, accepted_ids, commit_pos, cache_len and status are
 * exactly those of mars_accept_commit (taken once; one block table and one
 * length per sequence serve every layer). k_new, v_new
 * [n_layers, S, B, n_kv_heads, head_dim]; k_cache [n_layers, pages, Hkv, page,
 * d], v_cache [n_layers, pages, Hkv, d, page]: layer l of each is laid out as
 * in mars_accept_commit, and rows r < n of layer l of k_new/v_new go to layer
 * l of the caches. Two launches on `stream`: the decision (which advances
 * cache_len and writes commit_pos), then one workgroup per (sequence, layer)
 * that copies the rows commit_pos names. Limits as mars_accept_commit, and
 * 1 <= n_layers <= 65535.
 */
int mars_accept_commit_layers(const float* p_max, const int32_t* top_id, const float* tau,
                              const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* block_table, int32_t* cache_len,
                              int32_t* n_accepted, int32_t* accepted_ids, int32_t* commit_pos,
                              int32_t n_layers, int32_t S, int32_t B, int32_t n_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t max_pages,
                              int32_t num_pages, int32_t dtype, int32_t* status, void* stream);

/* Human-readable text for a MARS_* return code. */
const char* mars_strerror(int code);

/* Library version, as major * 10000 + minor * 100 + patch. */
int mars_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MARS_H_ */
