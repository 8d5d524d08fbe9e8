// KV append: the newest tokens' K and V rows into their slots of the paged
// HND cache ("GPT OSS" model notes, section 3: each layer's (K, V) are
// appended to the KV cache before the attention step; section 11: paged K/V
// per layer, in pages that the table maps).
//
// Token i of the n_b new tokens of sequence b sits at position
// p = L_b - n_b + i (the lengths already count the new tokens) and goes to
// page block_table[b][p / 16], slot p % 16, of every KV head.  The work is a
// scatter of rows of d elements, one thread per 16-byte chunk.  A wave takes
// the rows of one KV head for 64 / (row chunks) consecutive new tokens, so
// that when they are consecutive positions of one page (the usual case) its
// stores fill one contiguous stretch of that page's head slab; its loads
// read whole rows.
#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

struct AppendArgs {
    const u32x4_t *__restrict__ k_new;   // [total][Hkv][row_chunks]
    const u32x4_t *__restrict__ v_new;
    u32x4_t *__restrict__ k_cache;       // [pages][Hkv][16][row_chunks]
    u32x4_t *__restrict__ v_cache;
    const int32_t *__restrict__ block_table;
    const int32_t *__restrict__ seq_lens;
    const int32_t *__restrict__ cu_new;  // [B + 1], or NULL: one new token per sequence
    int num_seqs, num_kv_heads, max_pages, row_chunks;
    int tokens_per_wave;  // 64 / row_chunks
    int total_new;
    long long total_threads;
};

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void append_kv(AppendArgs a)
{
    const long long i = (long long)blockIdx.x * kAppendThreads + threadIdx.x;
    if (i >= a.total_threads)
        return;
    // i = ((token block * Hkv + g) * tokens_per_wave + token in block) * row_chunks + c
    const int c = (int)(i % a.row_chunks);
    const long long r = i / a.row_chunks;
    const int t_in = (int)(r % a.tokens_per_wave);
    const long long bg = r / a.tokens_per_wave;
    const int g = (int)(bg % a.num_kv_heads);
    const int t = (int)(bg / a.num_kv_heads) * a.tokens_per_wave + t_in;
    if (t >= a.total_new)
        return;  // past the last token of a partial block
    const size_t src = ((size_t)t * a.num_kv_heads + g) * a.row_chunks + c;
    int b = t, n = 1, first = t;
    if (a.cu_new) {
        // the sequence of token t: the last b with cu_new[b] <= t (empty
        // sequences share their offset with the next one and are skipped)
        int lo = 0, hi = a.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu_new[mid] <= t)
                lo = mid;
            else
                hi = mid - 1;
        }
        b = lo;
        first = a.cu_new[b];
        n = a.cu_new[b + 1] - first;
    }
    const int pos = a.seq_lens[b] - n + (t - first);
    const int page = a.block_table[(size_t)b * a.max_pages + (pos >> 4)];
    const size_t dst = (((size_t)page * a.num_kv_heads + g) * 16 + (pos & 15)) * a.row_chunks + c;
    a.k_cache[dst] = a.k_new[src];
    a.v_cache[dst] = a.v_new[src];
}

}  // namespace

hipError_t launch_append_kv(int elem_bytes, int num_seqs, int num_kv_heads, int head_dim,
                            int max_pages_per_seq, int total_new, const void *k_new,
                            const void *v_new, const int32_t *block_table,
                            const int32_t *seq_lens, const int32_t *cu_seqlens_new,
                            void *k_cache, void *v_cache, hipStream_t stream)
{
    if (total_new == 0 || num_seqs == 0)
        return hipSuccess;
    AppendArgs a;
    a.k_new = (const u32x4_t *)k_new;
    a.v_new = (const u32x4_t *)v_new;
    a.k_cache = (u32x4_t *)k_cache;
    a.v_cache = (u32x4_t *)v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.cu_new = cu_seqlens_new;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.max_pages = max_pages_per_seq;
    a.row_chunks = head_dim * elem_bytes / 16;  // 8, 16 or 32
    a.tokens_per_wave = 64 / a.row_chunks;
    a.total_new = total_new;
    const long long token_blocks = (total_new + a.tokens_per_wave - 1) / a.tokens_per_wave;
    a.total_threads = token_blocks * num_kv_heads * 64;
    const long long blocks = (a.total_threads + kAppendThreads - 1) / kAppendThreads;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(append_kv, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn
