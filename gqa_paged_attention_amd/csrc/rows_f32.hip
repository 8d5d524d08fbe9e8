// fp32 sink attention, one wave per (query token, query head), full rows.
//
// The fp32 dtype exists for exact-precision checks at small sizes, so this
// path favours plainness over speed: no split of the KV range and no matrix
// cores.  Per row it runs the online softmax of "GPT-OSS on day 0" (section
// "Sink Attention": running maximum and sum over blocks of the KV length) and
// folds the sink into the final normalisation ("GPT OSS" model notes, sections
// 3 and 4.1: the sink joins the maximum and the sum, with a zero value).
//
// Lane j scores key kb + j of a 64-key block (its own dot product over the
// head dimension, q staged in LDS); the block's weights are then broadcast
// with shuffles while lane c accumulates value dimensions c, c + 64.
#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

struct RowsArgs {
    const float *__restrict__ q;
    const float *__restrict__ k_cache;
    const float *__restrict__ v_cache;
    const int32_t *__restrict__ block_table;
    const int32_t *__restrict__ seq_lens;
    const int32_t *__restrict__ cu_seqlens_q;  // NULL: one query per sequence
    const float *__restrict__ sinks;
    float *__restrict__ out;
    int num_seqs, num_q_heads, num_kv_heads, group, max_pages;
    int window;  // sliding window W: keys p - W + 1 .. p (0: none)
    float scale_log2;
};

template <int D>
__global__ __launch_bounds__(64) void rows_f32(RowsArgs a)
{
    const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
    int b = t, q_len = 1, i = 0;
    if (a.cu_seqlens_q) {
        int lo = 0, hi = a.num_seqs - 1;  // last b with cu[b] <= t
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu_seqlens_q[mid] <= t)
                lo = mid;
            else
                hi = mid - 1;
        }
        b = lo;
        q_len = a.cu_seqlens_q[b + 1] - a.cu_seqlens_q[b];
        i = t - a.cu_seqlens_q[b];
    }
    const int L = a.seq_lens[b];
    const int n_vis = max(L - q_len + i + 1, 0);
    // oldest visible key ("GPT OSS" model notes, section 4.1: local window)
    const int k_lo = (a.window > 0 && n_vis > a.window) ? n_vis - a.window : 0;
    const int g = h / a.group;

    __shared__ float sq[D];
    const float *qrow = a.q + ((size_t)t * a.num_q_heads + h) * D;
    for (int c = lane; c < D; c += 64)
        sq[c] = qrow[c];
    __syncthreads();

    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    constexpr int kPer = D / 64;
    float acc[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        acc[j] = 0.f;
    float m = kNegInf, l = 0.f;

    for (int kb = k_lo; kb < n_vis; kb += 64) {
        const int key = kb + lane;
        float x = kNegInf;
        if (key < n_vis) {
            const float *krow =
                a.k_cache + (((size_t)bt[key >> 4] * a.num_kv_heads + g) * 16 + (key & 15)) * D;
            float dot = 0.f;
#pragma unroll 8
            for (int c = 0; c < D; ++c)
                dot = fmaf(sq[c], krow[c], dot);
            x = dot * a.scale_log2;
        }
        const float m_new = fmaxf(m, wave_max(x));  // finite: the block has a key
        const float alpha = exp2_fast(m - m_new);
        const float p = exp2_fast(x - m_new);
        l = l * alpha + wave_sum(p);
        m = m_new;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            acc[j] *= alpha;
        const int nk = min(64, n_vis - kb);
        for (int jj = 0; jj < nk; ++jj) {
            const float pj = __shfl(p, jj, 64);
            const int kj = kb + jj;
            const float *vrow =
                a.v_cache + (((size_t)bt[kj >> 4] * a.num_kv_heads + g) * 16 + (kj & 15)) * D;
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                acc[j] = fmaf(pj, vrow[lane + 64 * j], acc[j]);
        }
    }

    const float sink2 = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
    const float M = fmaxf(m, sink2);
    float scale = 0.f;
    if (M != kNegInf) {
        const float f = m == kNegInf ? 0.f : exp2_fast(m - M);
        const float den = l * f + (sink2 == kNegInf ? 0.f : exp2_fast(sink2 - M));
        scale = den > 0.f ? f / den : 0.f;
    }
    float *orow = a.out + ((size_t)t * a.num_q_heads + h) * D;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        orow[lane + 64 * j] = acc[j] * scale;
}

template <int D>
hipError_t launch_d(const RowsArgs &a, int total_q, hipStream_t stream)
{
    hipLaunchKernelGGL(rows_f32<D>, dim3(total_q, a.num_q_heads), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rows_f32(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int max_pages_per_seq, int total_q, const void *q,
                           const void *k_cache, const void *v_cache, const int32_t *block_table,
                           const int32_t *seq_lens, const int32_t *cu_seqlens_q,
                           const float *sinks, float scale, int window, void *out,
                           hipStream_t stream)
{
    if (total_q == 0 || num_seqs == 0)
        return hipSuccess;
    RowsArgs a;
    a.q = (const float *)q;
    a.k_cache = (const float *)k_cache;
    a.v_cache = (const float *)v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.cu_seqlens_q = cu_seqlens_q;
    a.sinks = sinks;
    a.out = (float *)out;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.max_pages = max_pages_per_seq;
    a.window = window;
    a.scale_log2 = scale * kLog2e;
    return head_dim == 64 ? launch_d<64>(a, total_q, stream) : launch_d<128>(a, total_q, stream);
}

}  // namespace attn
