/*
 * attn_sinks.h -- C ABI of the MI355X (gfx950) library for grouped-query
 * attention over a paged KV cache with per-head attention sinks.
 *
 * The operation (both entry points compute it; decode is the case of one
 * query token per sequence):
 *
 *   Each query head h owns a sink logit that joins the softmax as a virtual
 *   token: it takes part in the maximum and in the sum of exponentials and
 *   contributes a zero value vector ("GPT OSS" model notes, TensorSharp
 *   docs/models/gptoss.md, sections 1, 3 "Forward graph" and 4.1; the
 *   "GPT-OSS on day 0" post, section "Sink Attention").  With G = Hq / Hkv,
 *   query head h reads KV head g = h / G (GQA, model notes section 4.1).
 *   For query token i of sequence b (Lq_b query tokens, L_b visible keys,
 *   the query tokens being the last Lq_b of them):
 *
 *     p   = L_b - Lq_b + i                      causal, aligned to the end
 *     s_j = scale * <q_i,h , K_b,g[j]>          j = 0 .. p
 *     m   = max(max_j s_j, sink_h)
 *     out = sum_j e^(s_j - m) V_b,g[j] / (sum_j e^(s_j - m) + e^(sink_h - m))
 *
 *   The scale multiplies q.k only; the sink enters unscaled.  A sink of -inf
 *   (or sinks == NULL) is plain softmax attention.  A row with no visible key
 *   and a -inf sink yields 0.
 *
 * KV page layout (HND, "Hosting Qwen on Blackwell": heads major, the tokens of
 * one head contiguous):
 *
 *   k_cache, v_cache : [num_pages][num_kv_heads][page_size][head_dim]
 *   token j of sequence b, KV head g lives at
 *     cache[block_table[b * max_pages_per_seq + j / page_size]][g][j % page_size][:]
 *   Slots past a sequence's end may hold anything (NaN included); they are
 *   never read into a result.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers except where noted; sizes are host ints.
 *   - dtype is ATTN_DTYPE_F32 or ATTN_DTYPE_BF16 and applies to q, k_cache,
 *     v_cache and out together.  sinks are always fp32.
 *   - All tensors are dense and row-major without padding.  q, k_cache,
 *     v_cache, out and the workspace must be 16-byte aligned; the int32 and
 *     fp32 side arrays 4-byte aligned.
 *   - stream is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; the caller keeps every buffer alive until the stream
 *     has passed the call.  The library allocates nothing, frees nothing and
 *     keeps no pointer after returning (attn_sinks_decode_noalloc uses a
 *     fixed scratch of its own instead), never synchronises and never copies
 *     device data to the host, so calls can be captured into a HIP graph.
 *   - Arguments are checked on the host before anything is enqueued; a
 *     nonzero return value means nothing was enqueued, except ATTN_ERR_HIP,
 *     which reports a failed launch.  Device data (page ids, lengths, query
 *     offsets) is not checked: page ids must lie in [0, num_pages), every
 *     0 <= L_b <= max_seq_len, Lq_b <= L_b, and cu_seqlens_q must be
 *     non-decreasing from 0 to total_q.  Violations are undefined behaviour.
 *   - Faults of the device work surface at the caller's next synchronisation.
 *   - Calls are re-entrant; the library's only state is a read-once cache of
 *     debug environment settings and, for attn_sinks_decode_noalloc only,
 *     a fixed device scratch array per GPU (see there).
 */
#ifndef ATTN_SINKS_H
#define ATTN_SINKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_dtype {
    ATTN_DTYPE_F32 = 0,
    ATTN_DTYPE_BF16 = 1
};

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                     */
    ATTN_ERR_SHAPE = 2,       /* sizes inconsistent or out of range             */
    ATTN_ERR_UNSUPPORTED = 3, /* dtype / head_dim / page_size / group size      */
    ATTN_ERR_WORKSPACE = 4,   /* decode workspace smaller than required         */
    ATTN_ERR_ALIGN = 5,       /* a pointer is not aligned as required          */
    ATTN_ERR_HIP = 6,         /* the HIP runtime rejected a launch              */
    ATTN_ERR_SCRATCH = 7      /* needs more than attn_sinks_decode_noalloc's
                                 fixed scratch                                 */
};

/* Supported: head_dim 64 or 128; page_size 16; Hq % Hkv == 0 with
 * Hq / Hkv <= 16; dtype f32 or bf16.  Other values return
 * ATTN_ERR_UNSUPPORTED. */

/*
 * attn_sinks_decode_workspace_bytes -- bytes of device scratch that
 * attn_sinks_decode needs for these sizes (split-KV partial results: one fp32
 * running max, one fp32 running sum and head_dim fp32 weighted values per
 * piece and query head; the layout is given with attn_sinks_decode_merge).
 * Returns 0 for sizes that attn_sinks_decode would reject or that need no
 * scratch (max_seq_len == 0).  Depends on host integers only.
 */
size_t attn_sinks_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int max_seq_len);

/*
 * attn_sinks_decode -- one query token per sequence ("decode"), split along
 * the KV length and merged: each split keeps a running maximum and sum
 * ("GPT-OSS on day 0", section "Sink Attention": online softmax with a
 * running max and scale, parallel over heads and over the KV length), and
 * the sink is folded in once, in the final merge of the splits, so it is
 * counted exactly once however the KV range was split.  bf16 calls with
 * max_seq_len <= 512 take one direct pass instead (one wave per sequence and
 * KV head over all its keys, the sink folded at its end); the workspace is
 * still checked but then not touched.
 *
 *   q            [num_seqs][num_q_heads][head_dim]          dtype
 *   k_cache      [num_pages][num_kv_heads][page_size][head_dim] dtype
 *   v_cache      same shape as k_cache
 *   block_table  [num_seqs][max_pages_per_seq] int32 page ids
 *   seq_lens     [num_seqs] int32 visible keys L_b (the new token included)
 *   sinks        [num_q_heads] fp32, or NULL for "no sink" (-inf)
 *   scale        softmax scale applied to q.k (finite)
 *   out          [num_seqs][num_q_heads][head_dim]          dtype (written)
 *   workspace    device scratch of workspace_bytes bytes, at least
 *                attn_sinks_decode_workspace_bytes(...); contents on entry do
 *                not matter and are overwritten.
 *   max_seq_len  host upper bound of every seq_lens[b]; must not exceed
 *                max_pages_per_seq * page_size.
 */
int attn_sinks_decode(int dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int page_size, int num_pages, int max_pages_per_seq, int max_seq_len,
                      const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_table, const int32_t *seq_lens, const float *sinks,
                      float scale, void *out, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * The two passes of attn_sinks_decode, callable on their own (bf16 only for
 * the first pass).  attn_sinks_decode is exactly partials followed by merge
 * on the same stream with the same sizes, except for bf16 calls with
 * max_seq_len <= 512: those run one direct pass (one wave per sequence and
 * KV head over all its keys, no workspace touched), whose results meet the
 * same tolerance but need not equal the two passes' bits.  Running them separately lets a
 * caller time or overlap the passes, or combine partial results computed
 * elsewhere (for example over a KV range held by another device), since the
 * merge reads nothing but the workspace.
 *
 * Workspace layout.  Units are 32-token blocks of one sequence, numbered in
 * sequence order; there are U = sum_b ceil(L_b / 32) of them.  The split pass
 * runs W workgroups per group of up to 4 KV heads (W depends only on
 * num_seqs, num_kv_heads and max_seq_len); workgroup w takes units
 * [floor(w U / W), floor((w+1) U / W)) for every KV head of its group.  The
 * part of sequence b covered by workgroup w is stored in slot b + w, for all
 * query heads (slots = num_seqs + W):
 *   float ml [slots][num_q_heads][2]   running max in base-2 units
 *                                      (scale*q.k*log2 e) and the sum of
 *                                      2^(s_j - max) over the piece
 *   float acc[slots][num_q_heads][head_dim], starting at the first multiple
 *                                      of 4 floats after ml: the sum of
 *                                      2^(s_j - max) * V[j]
 * Only slots of pieces that exist are written and read; the byte count is
 * attn_sinks_decode_workspace_bytes.
 *
 * attn_sinks_decode_partials -- the split pass (dtype must be
 * ATTN_DTYPE_BF16); arguments as for attn_sinks_decode.  No sink is involved.
 */
int attn_sinks_decode_partials(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                               int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                               int max_seq_len, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_table,
                               const int32_t *seq_lens, float scale, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * attn_sinks_decode_merge -- the merge pass: for each (sequence, head)
 * combine the pieces' partial results with the sink, counted once
 * ("GPT-OSS on day 0", section "Sink Attention"):
 *   M = max(max_p m_p, sink * log2(e))
 *   out = sum_p acc_p 2^(m_p - M) / (sum_p l_p 2^(m_p - M) + 2^(sink*log2(e) - M))
 * and write out [num_seqs][num_q_heads][head_dim] in dtype (f32 or bf16).
 * The workspace is read only.
 */
int attn_sinks_decode_merge(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                            int head_dim, int max_seq_len, const int32_t *seq_lens,
                            const float *sinks, const void *workspace, size_t workspace_bytes,
                            void *out, void *stream);

/*
 * attn_sinks_prefill -- ragged batch of query chunks with causal masking
 * (model notes section 3: causal mask before the sink softmax).  The chunk of
 * sequence b is query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and sits at
 * the end of that sequence's L_b visible keys, so the rows of a chunk over a
 * cached prefix see the whole prefix.  The sink is folded into each row's
 * final normalisation.
 *
 *   q             [total_q][num_q_heads][head_dim]          dtype
 *   k_cache/v_cache, block_table, sinks, scale: as for decode
 *   seq_lens      [num_seqs] int32 visible keys L_b, chunk included
 *   cu_seqlens_q  [num_seqs + 1] int32 query offsets, 0 .. total_q
 *   out           [total_q][num_q_heads][head_dim]          dtype (written)
 *   max_q_len     host upper bound of every chunk length Lq_b
 *   max_seq_len   host upper bound of every L_b (<= max_pages_per_seq*page_size)
 */
int attn_sinks_prefill(int dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int page_size, int num_pages, int max_pages_per_seq, int total_q,
                       int max_q_len, int max_seq_len, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *block_table, const int32_t *seq_lens,
                       const int32_t *cu_seqlens_q, const float *sinks, float scale, void *out,
                       void *stream);

/*
 * Sliding-window variants.  The "GPT OSS" model notes give the model's even
 * layers a local attention window (section 4.1: SWA, window 128 by default)
 * and pass the per-layer window with each call into the paged kernel
 * (section 11).  With window = W > 0 the query at position p sees only the
 * keys at positions p - W + 1 .. p (its own included); the sink stays in
 * every row's softmax whatever the window:
 *
 *     s_j = scale * <q_i,h , K_b,g[j]>          j = max(0, p - W + 1) .. p
 *
 * and the rest of the definition above is unchanged.  window = 0 means no
 * window: these calls then run exactly the code of attn_sinks_decode and
 * attn_sinks_prefill and return bit-identical results.  A window of at least
 * max_seq_len also leaves every row whole and gives the same bits.  window <
 * 0 returns ATTN_ERR_SHAPE.  All other arguments, the workspace of the decode
 * (size from attn_sinks_decode_workspace_bytes, which covers every window),
 * ownership, checks and errors are as for the unwindowed calls.
 *
 * Decode reads only the blocks of each sequence that hold its last W keys;
 * bf16 with 0 < W <= 512 and W < max_seq_len runs one wave per (sequence,
 * KV head) over them and writes the output directly (the workspace is then
 * not touched).  bf16 prefill with 0 < W < max_seq_len at head_dim 64 and a
 * group size divisible by 4 runs on the causal prefill's pipeline over the
 * tiles its rows' windows reach; other shapes run a kernel in which each
 * wave streams the few blocks its rows need straight from the paged cache.
 *
 * Pages a window no longer reaches may be released: with W > 0, the page
 * table entries of sequence b below entry (L_b - Lq_b - W + 1) / 16 (decode:
 * (L_b - W) / 16; integer division, negative meaning none) are never read,
 * nor the pages they name, so they may hold any value, invalid page ids
 * included.  The fp32 path reads only the keys each row sees as well.
 */
int attn_sinks_decode_window(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                             int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                             int max_seq_len, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_table,
                             const int32_t *seq_lens, const float *sinks, float scale, int window,
                             void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_sinks_decode_noalloc -- attn_sinks_decode_window without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The split pass's partial results go to a fixed scratch array inside the
 * library instead: 32 MiB of device memory per GPU the library runs on,
 * held until the process ends.  The call itself allocates and frees
 * nothing; its first call on a device looks up that device's copy of the
 * array (the current device, hipGetDevice; the stream must belong to it).
 *
 * Arguments, results, checks and errors are those of
 * attn_sinks_decode_window (window 0: attn_sinks_decode), with the same bits.
 * A call whose workspace size (attn_sinks_decode_workspace_bytes of its
 * sizes) exceeds 32 MiB returns ATTN_ERR_SCRATCH with nothing enqueued; the
 * limit admits, for instance, 1800 sequences at 64 q heads and head_dim 64,
 * or 700 at 64 q heads and head_dim 128.  ATTN_ERR_HIP also reports a failed
 * lookup of the scratch.
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls on one stream
 * are ordered and safe, but two calls that may overlap on one GPU (different
 * streams without ordering between them) race and give undefined results.
 */
int attn_sinks_decode_noalloc(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                              int max_seq_len, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_table,
                              const int32_t *seq_lens, const float *sinks, float scale,
                              int window, void *out, void *stream);

int attn_sinks_prefill_window(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                              int total_q, int max_q_len, int max_seq_len, const void *q,
                              const void *k_cache, const void *v_cache,
                              const int32_t *block_table, const int32_t *seq_lens,
                              const int32_t *cu_seqlens_q, const float *sinks, float scale,
                              int window, void *out, void *stream);

/*
 * attn_sinks_mixed -- one batch of single-token decode sequences and causal
 * prefill chunks over one page pool: the step of continuous batching, which
 * serves concurrent requests, new prompts and running generations, in one
 * batched paged forward ("GPT OSS" model notes, section 11).  The operation
 * of each part is the one at the top of this file.
 *
 *   Sequences 0 .. num_decode_seqs - 1 are decodes: one query token each, in
 *   row b of q and out (so cu_seqlens_q[b] = b for b <= num_decode_seqs, a
 *   device-side precondition like those above), their lengths bounded by
 *   decode_max_seq_len.  Sequences num_decode_seqs .. +num_prefill_seqs - 1
 *   are prefill chunks: rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1,
 *   bounded by max_q_len and max_seq_len; total_q counts every row of both.
 *   seq_lens, block_table (max_pages_per_seq entries per sequence) and
 *   cu_seqlens_q cover the whole batch.
 *   The decode rows equal, bit for bit, attn_sinks_decode over the first
 *   num_decode_seqs sequences, and the chunk rows those of attn_sinks_prefill
 *   over the chunks alone (their rows, lengths and table rows taken as a
 *   batch of their own).  fp32 computes every row in one row-kernel launch;
 *   bf16 runs the two calls one after the other when either part is empty or
 *   the decode part is short enough for its direct pass, and otherwise the
 *   decode part's split pass and the prefill in one launch, the split pass's
 *   workgroups first in the grid (so the memory-bound pass runs beside the
 *   compute-bound prefill instead of before it), then the merge.
 *   workspace: attn_sinks_decode_workspace_bytes(num_decode_seqs, num_q_heads,
 *   num_kv_heads, head_dim, decode_max_seq_len) bytes.  Checks of both parts
 *   run before anything is enqueued; codes as for the two calls.
 */
int attn_sinks_mixed(int dtype, int num_decode_seqs, int num_prefill_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int page_size, int num_pages,
                     int max_pages_per_seq, int decode_max_seq_len, int total_q, int max_q_len,
                     int max_seq_len, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_table, const int32_t *seq_lens,
                     const int32_t *cu_seqlens_q, const float *sinks, float scale, void *out,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * KV append.  Before the attention step each layer appends the new tokens'
 * K and V to its KV cache ("GPT OSS" model notes, section 3, forward graph;
 * section 11: per-layer paged K/V).  The n_b new tokens of sequence b are its
 * last ones: seq_lens[b] = L_b already counts them, and token i of them
 * (i = 0 .. n_b - 1) sits at position p = L_b - n_b + i.  Its rows are
 * written to
 *     k_cache[block_table[b * max_pages_per_seq + p / page_size]][g][p % page_size][:]
 * (and v_cache likewise) for every KV head g.  Nothing else in the pool is
 * written.  The caller maps the pages (the table entries for the new
 * positions must be valid page ids).
 *
 *   k_new, v_new    [total_new][num_kv_heads][head_dim]  dtype, the new tokens
 *                   of sequence 0, then of sequence 1, ...
 *   cu_seqlens_new  [num_seqs + 1] int32 offsets of each sequence's new
 *                   tokens in k_new / v_new (0 .. total_new), or NULL for one
 *                   new token per sequence (then total_new must equal
 *                   num_seqs)
 *   k_cache, v_cache, block_table, seq_lens, max_seq_len: as for decode;
 *                   the caches are written.
 * Device preconditions (unchecked): n_b <= L_b and the written slots of two
 * tokens never coincide.  Other conventions as above.
 */
int attn_sinks_append_kv(int dtype, int num_seqs, int num_kv_heads, int head_dim, int page_size,
                         int num_pages, int max_pages_per_seq, int max_seq_len, int total_new,
                         const void *k_new, const void *v_new, const int32_t *block_table,
                         const int32_t *seq_lens, const int32_t *cu_seqlens_new, void *k_cache,
                         void *v_cache, void *stream);

/*
 * Rotary embedding fused into the KV append.  Each layer rotates Q and K
 * with NeoX-style RoPE under YaRN scaling before K is appended ("GPT OSS"
 * model notes, section 3, forward graph: origCtxLen 4096, freqScale =
 * 1 / RopeScale, beta_fast 32, beta_slow 1; section 4.1; section 11: the
 * positions come as an explicit array).  The notes give those parameters,
 * not the formula; the formula is YaRN's ("NTK-by-parts" interpolation with
 * attention scaling) in the form that takes beta_fast and beta_slow, the
 * arguments the notes' RoPEEx call names: the pair that turns beta times
 * within orig_ctx sits at the fractional index c(beta), and the blend is
 * linear in the pair index between c(beta_fast) and c(beta_slow):
 *
 *   theta_i = rope_base^(-2 i / head_dim)              i = 0 .. head_dim/2 - 1
 *   c(beta) = (head_dim / 2) ln(orig_ctx / (2 pi beta)) / ln(rope_base)
 *   ramp_i  = clamp((i - c(beta_fast)) / (c(beta_slow) - c(beta_fast)), 0, 1)
 *   f_i     = (1 - ramp_i) theta_i + ramp_i theta_i / rope_scale
 *   c       = 0.1 ln(rope_scale) + 1  (1 when rope_scale <= 1)
 *
 * and a row x at position p becomes, for every pair (i, i + head_dim/2):
 *
 *   y_i            = c (x_i cos(p f_i) - x_{i+d/2} sin(p f_i))
 *   y_{i+head_dim/2} = c (x_i sin(p f_i) + x_{i+d/2} cos(p f_i))
 *
 * rope_scale = 1 is plain RoPE.  The call rotates every query head of the
 * new tokens in q, in place, writes the rotated new K rows to their cache
 * slots and appends V unchanged, all as attn_sinks_append_kv places them.
 * Arithmetic is fp32 with the angle p f_i formed and reduced in fp64;
 * results are rounded to dtype (RNE).
 *
 *   q              [total_new][num_q_heads][head_dim] dtype, read and written
 *   positions      [total_new] int32 rotary position of each new token
 *                  (usually its cache position; any value is accepted)
 *   rope_base      > 0 and != 1; rope_scale > 0; orig_ctx > 0; when
 *                  rope_scale != 1, beta_fast > beta_slow > 0 (all finite),
 *                  else ATTN_ERR_SHAPE
 *   the rest       as for attn_sinks_append_kv (num_q_heads as for decode)
 * The new K rows in k_new are read only.  Device preconditions as for
 * attn_sinks_append_kv.
 */
int attn_sinks_rope_append(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                           int max_seq_len, int total_new, void *q, const void *k_new,
                           const void *v_new, const int32_t *positions, float rope_base,
                           float rope_scale, int orig_ctx, float beta_fast, float beta_slow,
                           const int32_t *block_table, const int32_t *seq_lens,
                           const int32_t *cu_seqlens_new, void *k_cache, void *v_cache,
                           void *stream);

/*
 * One layer's attention step as the forward graph of the model notes
 * (section 3) orders it: append the new tokens' K and V, then attend with
 * the sink, with an optional sliding window (0: none).  These are the
 * append above followed, on the same stream, by attn_sinks_decode_window or
 * attn_sinks_prefill_window; every check of both runs before anything is
 * enqueued.  Decode appends one token per sequence (k_new, v_new
 * [num_seqs][num_kv_heads][head_dim]); prefill appends the chunk's tokens,
 * whose offsets are cu_seqlens_q (k_new, v_new [total_q][num_kv_heads][head_dim]).
 */
int attn_sinks_decode_append(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                             int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                             int max_seq_len, const void *q, const void *k_new,
                             const void *v_new, void *k_cache, void *v_cache,
                             const int32_t *block_table, const int32_t *seq_lens,
                             const float *sinks, float scale, int window, void *out,
                             void *workspace, size_t workspace_bytes, void *stream);

int attn_sinks_prefill_append(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                              int total_q, int max_q_len, int max_seq_len, const void *q,
                              const void *k_new, const void *v_new, void *k_cache,
                              void *v_cache, const int32_t *block_table,
                              const int32_t *seq_lens, const int32_t *cu_seqlens_q,
                              const float *sinks, float scale, int window, void *out,
                              void *stream);

/*
 * Multi-token decode: a few new query tokens per sequence (Lq_b of them,
 * the last of its L_b keys), as when speculative or MTP draft tokens are
 * verified ("Hosting Qwen on Blackwell": decoding with speculative MTP
 * layers; "GPT-OSS on day 0": speculative and MTP decoders).  The result is
 * exactly that of attn_sinks_prefill on the same arguments (bottom-right
 * causal among the new tokens, sink in every row); the difference is the
 * kernel.  The split-KV decode passes run with the query rows of each KV
 * head packed GQA-style into the matrix columns (G x Lq rows share each K
 * and V block read, in layers of up to 64 rows at head_dim 64 and 32 at
 * head_dim 128; each further layer reads the blocks again), when
 *     dtype is bf16 and G * max_q_len <= 128;
 * other shapes run attn_sinks_prefill and need no workspace.
 *
 *   q, out        [total_q][num_q_heads][head_dim], rows as cu_seqlens_q says
 *   cu_seqlens_q  [num_seqs + 1] int32 query offsets (0 .. total_q)
 *   max_q_len     host upper bound of every Lq_b
 *   workspace     at least attn_sinks_decode_multi_workspace_bytes(...) bytes
 *                 (0 bytes, and NULL allowed, when that returns 0; the count
 *                 depends on the shape only, and fp32 calls never use it)
 * Everything else as for attn_sinks_prefill / attn_sinks_decode.  The
 * workspace layout is that of attn_sinks_decode_merge with max_q_len query
 * rows per slot: ml [slots][max_q_len][num_q_heads][2], acc likewise.
 */
size_t attn_sinks_decode_multi_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                               int head_dim, int max_seq_len, int max_q_len);

int attn_sinks_decode_multi(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                            int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                            int total_q, int max_q_len, int max_seq_len, const void *q,
                            const void *k_cache, const void *v_cache, const int32_t *block_table,
                            const int32_t *seq_lens, const int32_t *cu_seqlens_q,
                            const float *sinks, float scale, void *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * Ragged attention without a KV cache: each sequence's keys and values are
 * contiguous rows, as when an embedding model runs attention over ragged
 * inputs and instantiates no KV cache ("Fast embeddings on GPUs": ragged
 * attention kernels, no padding, no KV cache).  The same sink softmax as
 * above; with causal = 1 the rows of sequence b (Lq_b <= L_b) are the last
 * Lq_b positions of its L_b keys as in attn_sinks_prefill; with causal = 0
 * every row sees all L_b keys.  Also writes each row's log-sum-exp, so that
 * the result can be combined with attention states computed elsewhere.
 *
 *   q             [total_q][num_q_heads][head_dim]   bf16, rows as cu_seqlens_q says
 *   k, v          [total_kv][num_kv_heads][head_dim] bf16, sequence b's keys are rows
 *                 cu_seqlens_kv[b] .. cu_seqlens_kv[b+1]-1
 *   cu_seqlens_q, cu_seqlens_kv  [num_seqs + 1] int32 offsets from 0
 *   max_q_len, max_kv_len  host upper bounds of Lq_b and L_b
 *   causal        1 or 0
 *   sinks, scale  as above
 *   out           [total_q][num_q_heads][head_dim] bf16 (written)
 *   lse           [total_q][num_q_heads] fp32 (written), or NULL: the natural
 *                 log of the row's softmax denominator,
 *                 ln(sum_j e^(s_j) + e^(sink_h)), -inf for an empty row
 *                 without a sink.  With sinks == NULL it is the plain LSE of
 *                 the row's scores, which is what merging partial states
 *                 needs (fold the sink once, at the end).
 * bf16 only (ATTN_ERR_UNSUPPORTED otherwise); max_kv_len * num_kv_heads *
 * head_dim * 2 must stay below 2^31 (ATTN_ERR_SHAPE).  Other conventions
 * as above; nothing is allocated and no workspace is needed.
 */
int attn_sinks_ragged(int dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int total_q, int total_kv, int max_q_len, int max_kv_len, int causal,
                      const void *q, const void *k, const void *v, const int32_t *cu_seqlens_q,
                      const int32_t *cu_seqlens_kv, const float *sinks, float scale, void *out,
                      float *lse, void *stream);

/* Static English text for a status code (never NULL). */
const char *attn_sinks_status_string(int status);

/*
 * Debug settings, for diagnostics and tests; the first two give the same
 * results bit for bit, the third the same within rounding.  Defaults come
 * from the environment, read once:
 *   ATTN_DEBUG_PREFILL_ONE_HEAD  bf16 causal prefill with a group size
 *                                divisible by 4 gives each workgroup one
 *                                query head (256 rows at head_dim 64, 128 at
 *                                128) instead of four (64 or 32 rows each)
 *                                (ATTN_SINKS_PREFILL_ONE_HEAD=1)
 *   ATTN_DEBUG_PREFILL_WAIT_ALL  the prefill's waits for its direct K/V tile
 *                                loads take every load in flight instead of
 *                                leaving the next tile's loads outstanding
 *                                (ATTN_SINKS_PREFILL_WAIT_ALL=1)
 *   ATTN_DEBUG_PREFILL_WINDOW_STREAMED
 *                                a windowed bf16 prefill that would run on
 *                                the causal kernel's pipeline (head_dim 64,
 *                                group size divisible by 4) runs the kernel
 *                                whose waves stream their own blocks instead
 *                                (ATTN_SINKS_PREFILL_WINDOW_STREAMED=1); its
 *                                results differ in rounding only
 * attn_sinks_set_debug sets one (value 0 or nonzero) for the launches that
 * follow and returns its previous value, or -1 for an unknown setting.  Not
 * meant to be changed while other threads enqueue calls.
 */
enum attn_debug_setting {
    ATTN_DEBUG_PREFILL_ONE_HEAD = 0,
    ATTN_DEBUG_PREFILL_WAIT_ALL = 1,
    ATTN_DEBUG_PREFILL_WINDOW_STREAMED = 2
};
int attn_sinks_set_debug(int setting, int value);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int attn_sinks_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SINKS_H */
