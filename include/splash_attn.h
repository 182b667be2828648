/*
 * splash_attn.h -- C ABI of the block-verify decode attention library for
 * MI355X (gfx950): speculative-decoding verify attention over a paged KV cache
 * held as int8 codes with one fp16 scale per (token, kv head).
 *
 * What the method computes (the pages describe Splash, an inference engine):
 *  - A draft model proposes a block of tokens and the target model checks the
 *    whole block in one forward pass (Splash community summary on
 *    discuss.pytorch.kr, section "DFlash 2 speculative decoding as the default
 *    path"; bnskd.com article, "Tech core 1").  In attention this is: each of a
 *    request's d drafted rows attends causally over the cached context and the
 *    drafts up to and including itself.
 *  - The decode kernel reads the 8-bit KV cache directly and reuses every page
 *    across the query heads that share it and across the verify tokens
 *    (discuss.pytorch.kr summary, section "Metal kernels generated to shape";
 *    bnskd.com, "Tech core 2").
 *  - The cache is paged and indexed by prefix: requests with a common prefix
 *    reuse its pages (discuss.pytorch.kr summary, section "Batch scheduling and
 *    a memory budget fixed at start-up").  Here that is identical block_table
 *    entries.
 *  - Each request in a batch carries its own draft (same summary, DFlash 2
 *    section), so draft lengths are per request.
 *  - A decode step is submitted as one unit (same section), so no call here
 *    synchronises the host; memory is budgeted once at start-up (batching
 *    section), so no call allocates: the caller owns every buffer.
 *  - Kernels exist for exact shapes and ship precompiled with presets keyed by
 *    GPU core count, with no fallback path (summary, Metal-kernels and design
 *    sections): shapes outside the compiled set return SPLASH_ERR_UNSUPPORTED,
 *    and num_splits = 0 picks a preset from the device's compute-unit count.
 *
 * Conventions for every entry point:
 *  - Every buffer pointer is a DEVICE pointer owned by the caller.  bf16 and
 *    fp16 values travel as raw uint16_t bit patterns.  `stream` is a
 *    hipStream_t passed as void* (NULL = the default stream).
 *  - Calls only enqueue work on `stream`; they never synchronise and never
 *    allocate, and keep no per-call state.
 *  - Argument faults the host can see are returned synchronously as a status
 *    code and nothing is launched.  Values that live in device memory
 *    (context_lens, draft_lens, block_table entries) are trusted
 *    preconditions; violating them is undefined behaviour:
 *      0 <= draft_lens[b] <= T_max,  draft_lens[b] <= context_lens[b]
 *      context_lens[b] <= max_context_len (verify)
 *      ceil(context_lens[b] / P) <= max_pages_per_seq
 *      every block_table entry that is used lies in [0, num_pages)
 *      appended positions never land in a page another request shares
 *      every finite query element has |q| <= 65504 (verify multiplies q in
 *      binary16; elements below 2^-17 in magnitude are rounded to it, an
 *      absolute change under 2^-25)
 *  - Layouts (row-major, innermost last):
 *      q, out       bf16  [B][T_max][Hq][D]
 *      k_pool       int8  [num_pages][Hkv][P][D]   (a page is P token rows)
 *      v_pool       int8  [num_pages][Hkv][P/8][D][8]  (a page is two d-major
 *                                  tiles of 8 tokens: token p, dim d at
 *                                  ((p / 8) * D + d) * 8 + p % 8 in its page)
 *      k_scale,
 *      v_scale      fp16  [num_pages][Hkv][P]
 *      block_table  int32 [B][max_pages_per_seq]
 *      context_lens int32 [B]   tokens in the cache AFTER the draft block
 *      draft_lens   int32 [B]   draft t of request b is at position
 *                               context_lens[b] - draft_lens[b] + t
 *    Query head h reads kv head h / (Hq / Hkv).
 *  - Compiled shapes: P = 16; (D, Hq/Hkv) in {(64, 4), (128, 8), (256, 6)};
 *    T_max <= 16 for verify.  Append accepts D in {64, 128, 256} and any T_max.
 *  - q, out, k_pool, v_pool and the workspace must be 16-byte aligned.
 *  - Split partials of splash_verify_attn_partition and
 *    splash_verify_attn_splitk_merge (the exported pair, for callers that run
 *    context splits themselves, e.g. one split per device), in fp32 rows:
 *      part_o   fp32  [B][Hq][T_max][S][D]  the normalised partial row o_s of
 *                     draft t, query head h, split s
 *      part_lse fp32  [B][Hq][T_max][S]     its natural-log log-sum-exp lse_s
 *                     (-inf for a split with no visible key; its row is 0)
 *    Rows t >= draft_lens[b] are neither written nor read.
 *  - The workspace of splash_verify_attn is opaque: its size comes from
 *    splash_verify_attn_workspace_bytes and its contents are the library's.
 */
#ifndef SPLASH_ATTN_H
#define SPLASH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SPLASH_OK = 0,
    SPLASH_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad ratio, misalignment */
    SPLASH_ERR_UNSUPPORTED = 2,        /* shape outside the compiled set                     */
    SPLASH_ERR_WORKSPACE_TOO_SMALL = 3,
    SPLASH_ERR_LAUNCH = 4,             /* the HIP runtime refused a launch                   */
    SPLASH_ERR_DEVICE = 5              /* no usable device / device query failed             */
};

enum { SPLASH_SRC_F32 = 0, SPLASH_SRC_BF16 = 1 };

/*
 * splash_kv_append_int8 -- quantise new K and V rows into the int8 pools.
 * The write side of the 8-bit cache (the pages state only that the cache is
 * 8-bit -- summary, Metal-kernels section -- and that its precision is a
 * setting -- localai.co.kr 1.3.0 guide).  For each request b, token
 * t < draft_lens[b] and kv head g, the D source values x (fp32, or bf16
 * widened exactly) become
 *     amax  = max_d |x_d|                         (fp32)
 *     s16   = binary16 nearest to amax / 127      (fp32 division, ties to even)
 *     code  = clamp(rint(x_d / s), -127, 127)     (s = s16 widened; fp32; 0 if s == 0)
 * stored at position pos = context_lens[b] - draft_lens[b] + t:
 *     k_pool[page][g][pos % P][:], v_pool[page][g][:][pos % P],
 *     k_scale/v_scale[page][g][pos % P], page = block_table[b][pos / P].
 * Nothing else in the pools changes.  k_new, v_new: [B][T_max][Hkv][D], fp32
 * (src_dtype SPLASH_SRC_F32) or bf16 (SPLASH_SRC_BF16).  T_max is unbounded, so
 * one call can also fill a whole context.  Results are bit-exact, reproducible.
 */
int splash_kv_append_int8(const void* k_new, const void* v_new, int src_dtype,
                          int8_t* k_pool, int8_t* v_pool,
                          uint16_t* k_scale, uint16_t* v_scale,
                          const int32_t* block_table, int max_pages_per_seq,
                          const int32_t* context_lens, const int32_t* draft_lens,
                          int B, int T_max, int Hkv, int D, int P, int num_pages,
                          void* stream);

/*
 * splash_verify_attn_default_splits -- the split-K preset: how many context
 * splits one request's pages are cut into so that B * Hkv * splits work items
 * fill the device's compute units (presets keyed by core count, as the
 * summary's Metal-kernels section describes), with at least 8 pages a split
 * (4 at D = 256 up to 64 pages of context; one split at D = 64 up to 16
 * pages, where the merge launch costs more than it saves).  Returns >= 1, or a
 * negative status on bad arguments or a failed device query.
 */
int splash_verify_attn_default_splits(int B, int Hkv, int max_context_len, int P, int D);

/*
 * splash_verify_attn_workspace_bytes -- bytes of device workspace
 * splash_verify_attn needs for num_splits splits (0 when num_splits <= 1): the
 * split partials, held as fp16 tiles in the order the kernels produce them,
 * each (request, kv head, split) block holding its rows times a power of two
 * 2^jv chosen from its V scales (so that small and large V values both keep
 * binary16's precision), then, at 256-byte aligned offsets, their fp32
 * log-sum-exps and one int32 jv per block.  T_max does not change the size.
 */
size_t splash_verify_attn_workspace_bytes(int B, int T_max, int Hq, int D, int num_splits);

/*
 * splash_verify_attn -- block-verify attention.  For request b, draft
 * t < draft_lens[b], query head h (kv head g = h / (Hq/Hkv)), with
 * pos_t = context_lens[b] - draft_lens[b] + t:
 *     z_j  = sm_scale * sum_d q[b][t][h][d] * k_scale_j * k_code_j[d],  j = 0..pos_t
 *     out[b][t][h][:] = bf16( sum_j e^(z_j - max z) v_scale_j v_code_j[:] / sum_j e^(z_j - max z) )
 * with the codes and scales of token j read through block_table.  Rows
 * t >= draft_lens[b] of out are left untouched (draft_lens[b] = 0 makes request
 * b a no-op).  Every page of a (request, kv head) is read from memory once and
 * serves all Hq/Hkv query heads and all drafts of the request.
 * max_context_len: host-side upper bound on context_lens (sizes the grid).
 * num_splits: 0 = preset; > 0 forces that many context splits.  When more than
 * one split runs, workspace must hold splash_verify_attn_workspace_bytes(...)
 * bytes (workspace may be NULL when one split runs).  Accumulation is in fp32
 * (split partials pass through fp16, a relative rounding of at most 2^-11);
 * the result is deterministic for a given num_splits.  With more than one
 * split, B and Hkv must be at most 65535 (else SPLASH_ERR_UNSUPPORTED, checked
 * before anything is launched).
 */
int splash_verify_attn(const uint16_t* q, uint16_t* out,
                       const int8_t* k_pool, const int8_t* v_pool,
                       const uint16_t* k_scale, const uint16_t* v_scale,
                       const int32_t* block_table, int max_pages_per_seq,
                       const int32_t* context_lens, const int32_t* draft_lens,
                       int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                       int max_context_len, float sm_scale, int num_splits,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * splash_verify_attn_append -- the step that appends the drafted block to the
 * cache and verifies it, as one call: splash_kv_append_int8 and
 * splash_verify_attn fused (a decode step goes to the GPU as one unit:
 * discuss.pytorch.kr summary, section "DFlash 2 speculative decoding as the
 * default path").  k_new / v_new are the block's source rows, [B][T_max][Hkv][D]
 * in fp32 or bf16 as src_dtype (the arguments splash_kv_append_int8 takes);
 * block token t < draft_lens[b] sits at position context_lens[b] - draft_lens[b]
 * + t, whose page must be in block_table.  The workgroups whose split holds the
 * block's pages quantise its rows exactly as the append does and store them
 * into the pools' slots of those pages before they copy the pages (a split
 * of fewer than 24 pages holding the block starts its copies later for
 * that).  On return (stream order) the pools are byte-identical to those
 * splash_kv_append_int8 leaves, and out is bit-identical to splash_verify_attn's
 * after it with the same num_splits.  A block page id outside [0, num_pages)
 * is not written.  The pools are written, so nothing else may read or write
 * the block's pages during the call.
 * Errors as splash_verify_attn, plus SPLASH_ERR_INVALID_ARGUMENT for a null
 * k_new / v_new, an unknown src_dtype, or source rows not aligned to D / 64
 * elements.
 */
int splash_verify_attn_append(const void* k_new, const void* v_new, int src_dtype,
                              const uint16_t* q, uint16_t* out,
                              int8_t* k_pool, int8_t* v_pool,
                              uint16_t* k_scale, uint16_t* v_scale,
                              const int32_t* block_table, int max_pages_per_seq,
                              const int32_t* context_lens, const int32_t* draft_lens,
                              int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                              int max_context_len, float sm_scale, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * splash_verify_attn_noalloc -- splash_verify_attn for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no workspace argument; the split partials go to a scratch
 * array the library holds in device memory, SPLASH_NOALLOC_SCRATCH_BYTES bytes
 * on each GPU it runs on, kept until the process ends.  The call allocates
 * nothing.  A call whose splits need more than that
 * (splash_verify_attn_workspace_bytes(B, T_max, Hq, D, S) for the S it runs,
 * the preset when num_splits = 0) returns SPLASH_ERR_WORKSPACE_TOO_SMALL before
 * anything is launched, and SPLASH_ERR_DEVICE if the scratch's address cannot
 * be found.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (different streams without ordering between
 * them) race and give undefined results; calls on one stream do not.  The
 * scratch holds only partials each call writes before reading, so nothing in
 * it needs clearing.  Arguments, results and errors otherwise as
 * splash_verify_attn (same kernels: for the same num_splits the output is
 * bit-identical).
 */
#define SPLASH_NOALLOC_SCRATCH_BYTES (32u << 20)
int splash_verify_attn_noalloc(const uint16_t* q, uint16_t* out,
                               const int8_t* k_pool, const int8_t* v_pool,
                               const uint16_t* k_scale, const uint16_t* v_scale,
                               const int32_t* block_table, int max_pages_per_seq,
                               const int32_t* context_lens, const int32_t* draft_lens,
                               int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                               int max_context_len, float sm_scale, int num_splits, void* stream);

/*
 * splash_verify_attn_masked -- splash_verify_attn with a tree-shaped mask
 * inside the block instead of the causal chain.  DFlash 2's path selector picks
 * a coherent path among several candidate tokens per position (discuss.pytorch.kr
 * summary, DFlash 2 section); checking several candidates in one pass makes the
 * block a tree.  Draft t of request b attends to every key before the block
 * (positions < context_lens[b] - draft_lens[b]) and to the block key of draft u
 * exactly when bit u of block_masks[b][t] is set (uint32 [B][T_max], device;
 * bits u >= draft_lens[b] are ignored).  The chain masks (bits 0..t) give
 * splash_verify_attn's result bit for bit.  Precondition: bit t of
 * block_masks[b][t] is set (a draft sees itself).  Everything else as
 * splash_verify_attn; block_masks == NULL is SPLASH_ERR_INVALID_ARGUMENT.
 */
int splash_verify_attn_masked(const uint16_t* q, uint16_t* out,
                              const int8_t* k_pool, const int8_t* v_pool,
                              const uint16_t* k_scale, const uint16_t* v_scale,
                              const int32_t* block_table, int max_pages_per_seq,
                              const int32_t* context_lens, const int32_t* draft_lens,
                              const uint32_t* block_masks,
                              int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                              int max_context_len, float sm_scale, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * splash_verify_attn_window -- splash_verify_attn where every draft sees only
 * the last `window` keys up to and including itself: draft t at position
 * p = context_lens[b] - draft_lens[b] + t attends to keys p - window < j <= p.
 * Sliding-window attention is what the draft model uses so that its memory
 * stays bounded however long the context grows (discuss.pytorch.kr summary,
 * DFlash 2 section).  Only the pages inside a request's window are read: the
 * splits cover splash_verify_attn_window_tokens(max_context_len, T_max,
 * window, P) tokens, so size the workspace with
 * splash_verify_attn_workspace_bytes(B, T_max, Hq, D, S) for the S that
 * splash_verify_attn_default_splits (or num_splits) gives over that span.
 * window >= 1 (else SPLASH_ERR_INVALID_ARGUMENT); a window of at least the
 * context gives splash_verify_attn's result.  Everything else as
 * splash_verify_attn.
 */
int splash_verify_attn_window(const uint16_t* q, uint16_t* out,
                              const int8_t* k_pool, const int8_t* v_pool,
                              const uint16_t* k_scale, const uint16_t* v_scale,
                              const int32_t* block_table, int max_pages_per_seq,
                              const int32_t* context_lens, const int32_t* draft_lens,
                              int window,
                              int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                              int max_context_len, float sm_scale, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * splash_verify_attn_window_tokens -- the token span the splits of a windowed
 * call cover: min(max_context_len, P * (ceil((T_max + window - 1) / P) + 1)).
 * Negative status on bad arguments.
 */
int splash_verify_attn_window_tokens(int max_context_len, int T_max, int window, int P);

/*
 * splash_prefill_attn -- attention for a chunk of prefill tokens over the same
 * int8 paged cache.  The engine keeps a separate attention kernel for prefill
 * (large blocks) next to the verify one (discuss.pytorch.kr summary, section
 * "Metal kernels generated to shape"); the computation is the verify
 * definition with a long block: chunk token t < chunk_lens[b] of request b sits
 * at position p = context_lens[b] - chunk_lens[b] + t and attends to keys
 * 0..p.  The chunk's K and V must already be appended.  T_max is any length
 * (B * ceil(T_max / 16) <= 65535); q and out are bf16 [B][T_max][Hq][D]; rows
 * t >= chunk_lens[b] are left untouched.  The chunk runs as ceil(T_max / 16)
 * verify blocks of 16 tokens per request in one launch of each kernel, every
 * block attending over the cache up to its own last token (the pages a block
 * reads are read again by the later blocks of the chunk; the Infinity Cache
 * serves most of the repeats).  workspace: splash_prefill_attn_workspace_bytes
 * bytes for the same arguments (0: none needed).  Everything else as
 * splash_verify_attn; chunk_lens plays the part of draft_lens.
 */
int splash_prefill_attn(const uint16_t* q, uint16_t* out,
                        const int8_t* k_pool, const int8_t* v_pool,
                        const uint16_t* k_scale, const uint16_t* v_scale,
                        const int32_t* block_table, int max_pages_per_seq,
                        const int32_t* context_lens, const int32_t* chunk_lens,
                        int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                        int max_context_len, float sm_scale, int num_splits,
                        void* workspace, size_t workspace_bytes, void* stream);
size_t splash_prefill_attn_workspace_bytes(int B, int T_max, int Hq, int Hkv, int D, int P,
                                           int max_context_len, int num_splits);

/*
 * splash_verify_attn_partition -- the first half of splash_verify_attn on its
 * own: for each context split s (pages [s*L, (s+1)*L) with
 * L = splash_verify_attn_split_pages(...)), write for draft t < draft_lens[b]
 * and query head h the normalised partial row and its log-sum-exp
 *     o_s   = sum_{j in split, j <= pos_t} e^(z_j - m_s) v_hat_j / l_s
 *     lse_s = m_s + ln l_s      (natural log; -inf and a zero row when the
 *                                split holds no visible key)
 * into part_o and part_lse, fp32 rows in the layout described at the top of
 * this header ([B][Hq][T_max][S][D] and [B][Hq][T_max][S], S = num_splits).
 * For callers that combine partials themselves (for example across devices,
 * each running the splits of its own page range) with
 * splash_verify_attn_splitk_merge.  num_splits must be >= 1 (no preset here).
 * part_o 16-byte aligned.  The fp16 roundings of p and p * v_scale inside the
 * kernel are as in splash_verify_attn; the rows themselves are not rounded.
 */
int splash_verify_attn_partition(const uint16_t* q,
                                 const int8_t* k_pool, const int8_t* v_pool,
                                 const uint16_t* k_scale, const uint16_t* v_scale,
                                 const int32_t* block_table, int max_pages_per_seq,
                                 const int32_t* context_lens, const int32_t* draft_lens,
                                 int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                                 int max_context_len, float sm_scale, int num_splits,
                                 float* part_o, float* part_lse, void* stream);

/*
 * splash_verify_attn_split_pages -- pages per split L that the partition uses
 * for num_splits splits of a max_context_len context (a multiple of the
 * kernel's page group), and so the number of splits that hold any page:
 * ceil(ceil(max_context_len / P) / L).  Negative status on bad arguments.
 */
int splash_verify_attn_split_pages(int max_context_len, int P, int num_splits);

/*
 * splash_verify_attn_splitk_merge -- combine S context splits by their
 * log-sum-exps: for draft t < draft_lens[b] and query head h,
 *     M = max_s lse_s,  w_s = e^(lse_s - M)
 *     out[b][t][h][:] = bf16( sum_s w_s o_s[:] / sum_s w_s )
 * with part_o fp32 [B][Hq][T_max][S][D] (16-byte aligned) and part_lse fp32
 * [B][Hq][T_max][S] as splash_verify_attn_partition writes them, out bf16
 * [B][T_max][Hq][D] (8-byte aligned).  Splits are folded in ascending order, so
 * the same inputs give the same bits; a split with lse = -inf weighs nothing,
 * whatever its row holds.  Rows t >= draft_lens[b] of out are left untouched.
 * D in {64, 128, 256}; any T_max and Hq.
 */
int splash_verify_attn_splitk_merge(const float* part_o, const float* part_lse,
                                    uint16_t* out, const int32_t* draft_lens,
                                    int B, int T_max, int Hq, int D, int num_splits,
                                    void* stream);

/*
 * splash_verify_accept -- accept the verified part of a drafted block and roll
 * the cache back past the rest: the step after the verify pass.  The draft
 * model proposes a block, the target checks the whole block in one forward
 * pass, the final output is identical to autoregressive decoding, and
 * drafting, verification, acceptance and the state update run as one unit
 * (discuss.pytorch.kr summary, section "DFlash 2 speculative decoding as the
 * default path").  With greedy decoding that is, for request b and
 * d = draft_lens[b]:
 *   block_tokens[b][0]       the last committed token, block_tokens[b][1..d-1]
 *                            the drafts (the d tokens the verify pass attended);
 *   logits[b][t][:]          the target's logits for the token after block
 *                            position t (bf16, [B][T_max][V]);
 *   y_t = argmax_v logits[b][t][v]   the largest value, compared as the exact
 *                            value of the bf16 number (so -0 == +0); among equal
 *                            values the lowest id;
 *   accepted[b]   = 1 + the number of leading i < d - 1 with
 *                   block_tokens[b][i + 1] == y_i      (block tokens whose KV
 *                   entries stay in the cache, 1..d);
 *   next_token[b] = y_{accepted[b] - 1}               (the target's own token);
 *   context_lens[b] -= d - accepted[b]                 (in place).
 * The tokens the step emits, block_tokens[b][1 .. accepted[b] - 1] and then
 * next_token[b], are exactly those greedy autoregressive decoding emits.
 * d = 0 is a no-op: accepted[b] = 0, next_token[b] = -1, context_lens[b]
 * unchanged.  Rows t >= d of logits are not read.  Deterministic.
 * Arguments: logits 16-byte aligned, V a multiple of 8 in [8, 2^30];
 * 1 <= T_max <= 64 (SPLASH_ERR_UNSUPPORTED above); accepted and next_token are
 * int32 [B] outputs; context_lens is read and written.  Preconditions (trusted,
 * device memory): 0 <= draft_lens[b] <= T_max, draft_lens[b] <= context_lens[b],
 * no logit of a read row is NaN.
 * workspace: device memory of splash_verify_accept_workspace_bytes(B, T_max, V)
 * bytes, 16-byte aligned, caller-owned: the partial maxima of each row's
 * chunks (no need to clear it; calls that overlap in time must not share it).
 * Two kernel launches.
 */
size_t splash_verify_accept_workspace_bytes(int B, int T_max, int V);
int splash_verify_accept(const uint16_t* logits, const int32_t* block_tokens, const int32_t* draft_lens,
                         int32_t* context_lens, int32_t* accepted, int32_t* next_token,
                         int B, int T_max, int V, void* workspace, size_t workspace_bytes, void* stream);

/* Text for a status code (static storage, never NULL). */
const char* splash_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPLASH_ATTN_H */
