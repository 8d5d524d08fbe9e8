/*
 * oracle.c -- plain fp64 CPU reference for grouped-query attention over a
 * paged KV cache with per-head attention sinks.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library
 * under gqa_paged_attention_amd/) may include, link, load or call this file.
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * use it.  It shares no code, header or constant with the HIP kernels.
 *
 * What it computes (one query row r of sequence b, query head h):
 *
 *   "GPT OSS" model notes (TensorSharp docs/models/gptoss.md), section 1 and
 *   section 4.1: each head owns a learned sink logit that acts as a virtual
 *   token inside the softmax -- it takes part in the max and in the sum of
 *   exponentials but adds nothing to the weighted sum of values.  Section 3
 *   ("Forward graph") writes the steps: scores = Q K^T, causal mask,
 *   denominators = exp(scores - max) + exp(sink - max), weights = exp(scores
 *   - max) / denominators, out = weights x V.  The "GPT-OSS on day 0" post
 *   (section "Sink Attention") describes the same bias joining the softmax.
 *
 *   With G = Hq / Hkv, KV head g = floor(h / G) (GQA, section 4.1 of the
 *   model notes: NumKVHeads < NumHeads, consecutive heads share a KV head).
 *
 *   p      = L_b - Lq_b + r            (position of the query; bottom-right
 *                                       causal alignment, so a decode token
 *                                       sees every cached key)
 *   j0     = 0, or max(0, p - W + 1) with a sliding window of W > 0
 *   s_j    = scale * sum_c q[c] * K_b[j][c],   j = j0 .. p
 *
 *   Without the causal mask (the ragged, cache-free attention of encoder-style
 *   embedding models, "Fast embeddings on GPUs": ragged inputs, no KV cache)
 *   every row of sequence b sees all L_b keys: p = L_b - 1 for every row.
 *   m      = max(max_j s_j, sink_h)
 *   den    = sum_j exp(s_j - m) + exp(sink_h - m)
 *   out    = sum_j exp(s_j - m) * V_b[j] / den
 *
 *   Sliding window: the model notes (section 4.1, attention pattern; section
 *   11, a per-layer window passed with each call into the paged kernel) give
 *   even layers a local window of W = 128 positions.  Read here as: the query
 *   at position p sees the W most recent positions p - W + 1 .. p, itself
 *   included; the sink stays available whatever the window.
 *
 *   K_b[j] is read through the page table in HND page layout ("Hosting Qwen
 *   on Blackwell": KV caches laid out head-major with the tokens of a head
 *   contiguous):  k_cache[block_table[b][j / P]][g][j % P][0 .. d).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - the scale multiplies q.k only; the sink enters the softmax unscaled;
 *   - the sum over keys is implied by the softmax in the forward graph;
 *   - the virtual token's logit is the sink value and its value vector is 0;
 *   - an empty visible set with sink = -inf yields out = 0 (no NaN);
 *   - bf16 inputs are widened exactly (16-bit shift) before any arithmetic.
 *
 * Everything is fp64, computed in logical key order j = 0, 1, ... so that the
 * result does not depend on which physical pages hold the keys.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Exact widening of one stored element to fp64. */
static double widen(const void *base, size_t idx, int dtype)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Index of element 0 of logical token j of KV head g of sequence b. */
static size_t kv_row(const int32_t *block_table, int max_pages_per_seq, int b, int j, int g,
                     int num_kv_heads, int page_size, int head_dim)
{
    int32_t page = block_table[(size_t)b * max_pages_per_seq + j / page_size];
    return (((size_t)page * num_kv_heads + g) * page_size + (j % page_size)) * head_dim;
}

/* Sequence that owns query token t (cu_seqlens_q is non-decreasing). */
static int owner_seq(const int32_t *cu_seqlens_q, int num_seqs, int64_t t)
{
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (cu_seqlens_q[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

/*
 * oracle_attention_rows -- compute n_rows (query token, query head) outputs.
 *
 *   q            [total_q][Hq][d] in dtype (f32 or bf16 bits)
 *   k/v_cache    [num_pages][Hkv][page_size][d] in dtype
 *   block_table  [num_seqs][max_pages_per_seq] int32
 *   seq_lens     [num_seqs] visible KV length L_b (includes the new tokens)
 *   cu_seqlens_q [num_seqs + 1] query offsets (decode: 0, 1, 2, ...)
 *   sinks        [Hq] fp32, or NULL meaning every sink is -inf
 *   window       sliding window W (keys p - W + 1 .. p), or 0 for none
 *   causal       1: bottom-right causal mask; 0: every row sees all keys
 *   row_token    [n_rows] query token index t in [0, total_q)
 *   row_head     [n_rows] query head h in [0, Hq)
 *   out          [n_rows][d] fp64
 *   lse          [n_rows] fp64 natural-log denominator m + log(den), or NULL
 *
 * Returns 0 on success, nonzero on a bad argument or allocation failure.
 */
int oracle_attention_rows(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                          int head_dim, int page_size, int max_pages_per_seq,
                          const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *block_table, const int32_t *seq_lens,
                          const int32_t *cu_seqlens_q, const float *sinks, double scale,
                          int window, int causal, int64_t n_rows, const int64_t *row_token, const int32_t *row_head,
                          double *out, double *lse, int num_threads)
{
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        page_size <= 0 || num_q_heads % num_kv_heads != 0 || window < 0)
        return 1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16)
        return 1;
    const int group = num_q_heads / num_kv_heads;
    int max_len = 0;
    for (int b = 0; b < num_seqs; ++b)
        if (seq_lens[b] > max_len)
            max_len = seq_lens[b];
    int failed = 0;

#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif

#pragma omp parallel reduction(| : failed)
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)head_dim);
        double *acc = (double *)malloc(sizeof(double) * (size_t)head_dim);
        if (!scores || !qrow || !acc)
            failed = 1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (failed)
                continue;
            const int64_t t = row_token[r];
            const int h = row_head[r];
            const int b = owner_seq(cu_seqlens_q, num_seqs, t);
            const int q_len = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
            const int i = (int)(t - cu_seqlens_q[b]);
            const int pos = seq_lens[b] - q_len + i;
            /* the row's last visible key */
            const int last = causal ? pos : seq_lens[b] - 1;
            const int n_vis = last + 1 < 0 ? 0 : last + 1;
            const int j0 = (window > 0 && n_vis - window > 0) ? n_vis - window : 0;
            const int g = h / group;
            const double sink = sinks ? (double)sinks[h] : -INFINITY;

            for (int c = 0; c < head_dim; ++c)
                qrow[c] = widen(q, ((size_t)t * num_q_heads + h) * head_dim + c, dtype);

            /* pass 1: logits and their maximum, the sink included */
            double m = sink;
            for (int j = j0; j < n_vis; ++j) {
                const size_t row = kv_row(block_table, max_pages_per_seq, b, j, g,
                                          num_kv_heads, page_size, head_dim);
                double dot = 0.0;
                for (int c = 0; c < head_dim; ++c)
                    dot += qrow[c] * widen(k_cache, row + c, dtype);
                scores[j] = scale * dot;
                if (scores[j] > m)
                    m = scores[j];
            }

            /* pass 2: exponentials, denominator with the sink, weighted values */
            for (int c = 0; c < head_dim; ++c)
                acc[c] = 0.0;
            double den = 0.0;
            if (m != -INFINITY) {
                for (int j = j0; j < n_vis; ++j) {
                    const size_t row = kv_row(block_table, max_pages_per_seq, b, j, g,
                                              num_kv_heads, page_size, head_dim);
                    double e = exp(scores[j] - m);
                    den += e;
                    for (int c = 0; c < head_dim; ++c)
                        acc[c] += e * widen(v_cache, row + c, dtype);
                }
                den += exp(sink - m); /* the virtual token: logit = sink, value = 0 */
            }
            double *o = out + (size_t)r * head_dim;
            for (int c = 0; c < head_dim; ++c)
                o[c] = den > 0.0 ? acc[c] / den : 0.0;
            if (lse)
                lse[r] = den > 0.0 ? m + log(den) : -INFINITY;
        }
        free(scores);
        free(qrow);
        free(acc);
    }
    return failed;
}
