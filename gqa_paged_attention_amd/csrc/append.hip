// KV append: the newest tokens' K and V rows into their slots of the paged
// HND cache ("GPT OSS" model notes, section 3: each layer's (K, V) are
// appended to the KV cache before the attention step; section 11: paged K/V
// per layer, in pages that the table maps).
//
// Token i of the n_b new tokens of sequence b sits at position
// p = L_b - n_b + i (the lengths already count the new tokens) and goes to
// page block_table[b][p / 16], slot p % 16, of every KV head.  The work is a
// scatter of rows of d elements.  A workgroup takes a run of consecutive new
// tokens: its threads first issue the loads of the run (one contiguous
// stretch of the token-major source, 16 bytes a thread per pass), while one
// thread per token finds the token's sequence, position and page and leaves
// the destination row in LDS; after a barrier the stores follow.  The
// lookups' chain of dependent reads thus overlaps the streaming loads
// instead of preceding every 16-byte copy.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kAppendPasses = 8;                                  // 16-byte chunks per thread
constexpr int kAppendChunks = kAppendThreads * kAppendPasses;     // per workgroup and pass group
constexpr int kAppendMaxTokens = kAppendChunks / 8;               // rows have >= 8 chunks
static_assert(kAppendMaxTokens <= kAppendThreads, "one lookup thread per token");

struct AppendArgs {
    const u32x4_t *__restrict__ k_new;   // [total][Hkv][row_chunks]
    const u32x4_t *__restrict__ v_new;
    u32x4_t *__restrict__ k_cache;       // [pages][Hkv][16][row_chunks]
    u32x4_t *__restrict__ v_cache;
    const int32_t *__restrict__ block_table;
    const int32_t *__restrict__ seq_lens;
    const int32_t *__restrict__ cu_new;  // [B + 1], or NULL: one new token per sequence
    int num_seqs, num_kv_heads, max_pages;
    int tokens_per_block;
    int total_new;
};

// Destination row (in rows of the cache viewed as [pages * Hkv * 16][row])
// of head 0 of new token t.
__device__ __forceinline__ long long dest_row(const AppendArgs &a, int t)
{
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
    return ((long long)page * a.num_kv_heads) * 16 + (pos & 15);
}

template <int kRowChunks>
__global__ __launch_bounds__(kAppendThreads) void append_kv(AppendArgs a)
{
    __shared__ long long rows[kAppendMaxTokens];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * a.tokens_per_block;
    const int nt = min(a.tokens_per_block, a.total_new - t0);
    const int per_token = a.num_kv_heads * kRowChunks;
    const int total = nt * per_token;  // chunks of this workgroup, per tensor
    const size_t src0 = (size_t)t0 * per_token;

    u32x4_t kx[kAppendPasses], vx[kAppendPasses];
#pragma unroll
    for (int u = 0; u < kAppendPasses; ++u) {
        const int j = u * kAppendThreads + tid;
        if (j < total) {
            kx[u] = __builtin_nontemporal_load(a.k_new + src0 + j);
            vx[u] = __builtin_nontemporal_load(a.v_new + src0 + j);
        }
    }
    if (tid < nt)
        rows[tid] = dest_row(a, t0 + tid);
    __syncthreads();

    // a row of more than kAppendChunks chunks in total (one token per
    // workgroup) takes further pass groups
    for (int base = 0;; base += kAppendChunks) {
#pragma unroll
        for (int u = 0; u < kAppendPasses; ++u) {
            const int j = base + u * kAppendThreads + tid;
            if (j < total) {
                const int tl = j / per_token;
                const int rem = j - tl * per_token;
                const int g = rem / kRowChunks;
                const int c = rem % kRowChunks;
                const size_t dst = (size_t)(rows[tl] + g * 16) * kRowChunks + c;
                a.k_cache[dst] = kx[u];
                a.v_cache[dst] = vx[u];
            }
        }
        if (base + kAppendChunks >= total)
            break;
#pragma unroll
        for (int u = 0; u < kAppendPasses; ++u) {
            const int j = base + kAppendChunks + u * kAppendThreads + tid;
            if (j < total) {
                kx[u] = __builtin_nontemporal_load(a.k_new + src0 + j);
                vx[u] = __builtin_nontemporal_load(a.v_new + src0 + j);
            }
        }
    }
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
    a.total_new = total_new;
    const int row_chunks = head_dim * elem_bytes / 16;  // 8, 16 or 32
    const long long per_token = (long long)num_kv_heads * row_chunks;
    if (per_token * total_new > 0x7fffffffLL)
        return hipErrorInvalidValue;
    // as many tokens as fill one pass group, but no fewer workgroups than
    // compute units while the tokens allow
    int tpb = (int)std::max<long long>(1, kAppendChunks / per_token);
    tpb = std::min(tpb, std::max(1, total_new / 256));
    a.tokens_per_block = tpb;
    const unsigned blocks = (unsigned)((total_new + tpb - 1) / tpb);
    switch (row_chunks) {
    case 8:
        hipLaunchKernelGGL(append_kv<8>, dim3(blocks), dim3(kAppendThreads), 0, stream, a);
        break;
    case 16:
        hipLaunchKernelGGL(append_kv<16>, dim3(blocks), dim3(kAppendThreads), 0, stream, a);
        break;
    case 32:
        hipLaunchKernelGGL(append_kv<32>, dim3(blocks), dim3(kAppendThreads), 0, stream, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace attn
