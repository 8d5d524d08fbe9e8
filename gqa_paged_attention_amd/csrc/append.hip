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

// Arguments of the fused rotate-and-append: the append's own (the head-0 row
// of each new token's slot) plus the rotation's.
struct RopeArgs {
    AppendArgs app;
    void *q;                  // [total_new][Hq][d], rotated in place
    const void *k_new, *v_new;
    void *k_cache, *v_cache;
    const int32_t *__restrict__ positions;  // [total_new]
    int num_q_heads;
    float mscale;             // YaRN's factor on q and k
    double freq[64];          // per-pair angular frequency (d/2 <= 64)
};

constexpr double kInv2Pi = 0.15915494309189533577;
constexpr double k2PiHi = 6.28318530717958623200;    // 2 pi rounded to double
constexpr double k2PiLo = 2.44929359829470635445e-16;  // 2 pi - k2PiHi

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

// Rotary embedding fused into the append ("GPT OSS" model notes, sections 3
// and 4.1: Q and K are rotated, NeoX-style with YaRN scaling, before K is
// appended; section 11: the positions come as an explicit array).  One
// workgroup per new token.  Its first d/2 threads compute the cosine and sine
// of the token's d/2 pairs -- the angle p * f_i in double, reduced by 2 pi in
// two parts, the sine and cosine of the remainder in float -- into LDS; then
// thread (h, sub) rotates the 16-byte chunks sub of both halves of head h
// (element i pairs with element i + d/2): every query head in place, the new
// K rows into their cache slots, and copies V as it is.
constexpr int kRopeThreads = 256;

template <typename T>
struct Vec16;  // one 16-byte chunk of a row
template <>
struct Vec16<uint16_t> {
    using type = u32x4_t;
    static constexpr int kElems = 8;
    static __device__ __forceinline__ void load(type v, float (&x)[8])
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(v[j] << 16);
            x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ type store(const float (&x)[8])
    {
        return type{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                    pack_bf16(x[6], x[7])};
    }
};
template <>
struct Vec16<float> {
    using type = f32x4_t;
    static constexpr int kElems = 4;
    static __device__ __forceinline__ void load(type v, float (&x)[4])
    {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            x[j] = v[j];
    }
    static __device__ __forceinline__ type store(const float (&x)[4])
    {
        return type{x[0], x[1], x[2], x[3]};
    }
};

template <int D, typename T>
__device__ __forceinline__ void rotate_row(const T *src, T *dst, int i0, const float *cs,
                                           const float *sn)
{
    using VT = Vec16<T>;
    constexpr int E = VT::kElems;
    float x1[E], x2[E], y1[E], y2[E];
    VT::load(*(const typename VT::type *)(src + i0), x1);
    VT::load(*(const typename VT::type *)(src + i0 + D / 2), x2);
#pragma unroll
    for (int j = 0; j < E; ++j) {
        y1[j] = x1[j] * cs[i0 + j] - x2[j] * sn[i0 + j];
        y2[j] = x1[j] * sn[i0 + j] + x2[j] * cs[i0 + j];
    }
    *(typename VT::type *)(dst + i0) = VT::store(y1);
    *(typename VT::type *)(dst + i0 + D / 2) = VT::store(y2);
}

template <int D, typename T>
__global__ __launch_bounds__(kRopeThreads) void rope_append(RopeArgs ra)
{
    using V = typename Vec16<T>::type;
    constexpr int kSub = D / 2 / Vec16<T>::kElems;  // threads per head
    constexpr int kHeadsPerPass = kRopeThreads / kSub;
    __shared__ float cs[D / 2], sn[D / 2];
    const AppendArgs &a = ra.app;
    const int t = blockIdx.x;
    const long long row = dest_row(a, t);  // cache row of head 0 (scalar loads, issued early)
    if (threadIdx.x < D / 2) {
        const int i = threadIdx.x;
        const double ang = (double)ra.positions[t] * ra.freq[i];
        const double k = rint(ang * kInv2Pi);
        const double r = fma(-k, k2PiLo, fma(-k, k2PiHi, ang));  // |r| <= pi (+ rounding)
        float s, c;
        sincosf((float)r, &s, &c);
        cs[i] = c * ra.mscale;
        sn[i] = s * ra.mscale;
    }
    __syncthreads();
    const int sub = threadIdx.x % kSub, hh = threadIdx.x / kSub;
    const int i0 = sub * Vec16<T>::kElems;
    T *q = (T *)ra.q + (size_t)t * ra.num_q_heads * D;
    for (int h = hh; h < ra.num_q_heads; h += kHeadsPerPass)
        rotate_row<D, T>(q + (size_t)h * D, q + (size_t)h * D, i0, cs, sn);
    const T *kn = (const T *)ra.k_new + (size_t)t * a.num_kv_heads * D;
    const T *vn = (const T *)ra.v_new + (size_t)t * a.num_kv_heads * D;
    T *kc = (T *)ra.k_cache, *vc = (T *)ra.v_cache;
    for (int h = hh; h < a.num_kv_heads; h += kHeadsPerPass) {
        const size_t dst = (size_t)(row + 16 * h) * D;
        rotate_row<D, T>(kn + (size_t)h * D, kc + dst, i0, cs, sn);
        *(V *)(vc + dst + i0) = *(const V *)(vn + (size_t)h * D + i0);
        *(V *)(vc + dst + i0 + D / 2) = *(const V *)(vn + (size_t)h * D + i0 + D / 2);
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

hipError_t launch_rope_append(int elem_bytes, int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_dim, int max_pages_per_seq, int total_new, void *q,
                              const void *k_new, const void *v_new, const int32_t *positions,
                              const double *freq, float mscale, const int32_t *block_table,
                              const int32_t *seq_lens, const int32_t *cu_seqlens_new,
                              void *k_cache, void *v_cache, hipStream_t stream)
{
    if (total_new == 0 || num_seqs == 0)
        return hipSuccess;
    RopeArgs r = {};
    AppendArgs &a = r.app;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.cu_new = cu_seqlens_new;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.max_pages = max_pages_per_seq;
    a.total_new = total_new;
    r.q = q;
    r.k_new = k_new;
    r.v_new = v_new;
    r.k_cache = k_cache;
    r.v_cache = v_cache;
    r.positions = positions;
    r.num_q_heads = num_q_heads;
    r.mscale = mscale;
    for (int i = 0; i < head_dim / 2; ++i)
        r.freq[i] = freq[i];
    const dim3 grid((unsigned)total_new);
    if (head_dim == 64 && elem_bytes == 2)
        hipLaunchKernelGGL((rope_append<64, uint16_t>), grid, dim3(kRopeThreads), 0, stream, r);
    else if (head_dim == 128 && elem_bytes == 2)
        hipLaunchKernelGGL((rope_append<128, uint16_t>), grid, dim3(kRopeThreads), 0, stream, r);
    else if (head_dim == 64)
        hipLaunchKernelGGL((rope_append<64, float>), grid, dim3(kRopeThreads), 0, stream, r);
    else if (head_dim == 128)
        hipLaunchKernelGGL((rope_append<128, float>), grid, dim3(kRopeThreads), 0, stream, r);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
