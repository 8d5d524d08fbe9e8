// Causal prefill for paged GQA attention with per-head sinks (bf16, gfx950).
//
// Each query row runs the online softmax of "GPT-OSS on day 0" (section
// "Sink Attention": running maximum and sum over blocks of keys) and the sink
// is folded into the row's final normalisation ("GPT OSS" model notes,
// sections 3 and 4.1).  The causal mask is aligned to the end of the visible
// keys, so a chunk over a cached prefix sees the whole prefix.
//
// Work decomposition: grid (q tiles, Hq, B), 256 threads.  A workgroup owns
// BM = 128 consecutive query rows of one query head of one sequence (heaviest
// tiles first); wave w owns rows 32w .. 32w+31 as two 16-row MFMA blocks.
// Keys are walked in tiles of BN = 64 (four 16-token HND page slabs):
//   - the workgroup copies the K tile to LDS row-major and the V tile to LDS
//     transposed ([dim][key]) -- each thread packs pairs of keys per dimension;
//   - S^T[16 keys x 16 rows] = K[16 x d] (LDS) * Q^T[d x 16] (registers),
//     16x16x32 bf16 MFMA; lane l then holds keys 4*(l/16)+i of row l%16;
//   - mask (diagonal and tail tiles only), row maximum over the 4 lane groups,
//     lazy rescale, p = 2^(s - m) in registers;
//   - O^T[16 dims x 16 rows] += V^T[16 dims x 32 keys] (LDS) * P^T (registers):
//     the S^T accumulators are already the P^T operand, and every row's
//     softmax state stays in the lane that owns the row.
#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;

struct PrefillArgs {
    const uint16_t *__restrict__ q;
    const uint16_t *__restrict__ k_cache;
    const uint16_t *__restrict__ v_cache;
    const int32_t *__restrict__ block_table;
    const int32_t *__restrict__ seq_lens;
    const int32_t *__restrict__ cu_seqlens_q;
    const float *__restrict__ sinks;
    uint16_t *__restrict__ out;
    int num_q_heads, num_kv_heads, group, max_pages, num_q_tiles;
    float scale_log2;
};

template <int D>
struct Smem {
    static constexpr int kKStride = D + 8;     // bf16 elements per K row (16 B pad)
    static constexpr int kVStride = kBN + 8;   // bf16 elements per V^T row (16 B pad)
    uint16_t k[kBN * kKStride];
    uint16_t vt[D * kVStride];
};

template <int D>
__device__ __forceinline__ void load_tile(Smem<D> &sm, const PrefillArgs &a,
                                          const int32_t *__restrict__ bt, int kv0, int L, int g)
{
    const int tid = threadIdx.x;
    constexpr size_t slab = 16 * D;
    // K: 16-byte chunks, row-major copy
    constexpr int kChunks = kBN * D / 8;
#pragma unroll
    for (int c = tid; c < kChunks; c += kThreads) {
        const int key = c / (D / 8), dc = c % (D / 8);
        const int t = kv0 + key;
        u32x4_t v = {0, 0, 0, 0};
        if (t < L) {
            const size_t base = ((size_t)bt[t >> 4] * a.num_kv_heads + g) * slab;
            v = *(const u32x4_t *)(a.k_cache + base + (t & 15) * D + dc * 8);
        }
        *(u32x4_t *)(&sm.k[key * Smem<D>::kKStride + dc * 8]) = v;
    }
    // V: pairs of keys x 8 dims, written transposed as (key 2p, key 2p+1) words
    constexpr int kPairs = (kBN / 2) * (D / 8);
#pragma unroll
    for (int c = tid; c < kPairs; c += kThreads) {
        const int kp = c % (kBN / 2), dc = c / (kBN / 2);
        const int t = kv0 + 2 * kp;
        u32x4_t v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
        if (t < L) {
            const size_t base = ((size_t)bt[t >> 4] * a.num_kv_heads + g) * slab;
            v0 = *(const u32x4_t *)(a.v_cache + base + (t & 15) * D + dc * 8);
        }
        if (t + 1 < L) {
            const size_t base = ((size_t)bt[(t + 1) >> 4] * a.num_kv_heads + g) * slab;
            v1 = *(const u32x4_t *)(a.v_cache + base + ((t + 1) & 15) * D + dc * 8);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t *row0 = (uint32_t *)&sm.vt[(dc * 8 + 2 * w) * Smem<D>::kVStride];
            uint32_t *row1 = (uint32_t *)&sm.vt[(dc * 8 + 2 * w + 1) * Smem<D>::kVStride];
            row0[kp] = pair_half(v0[w], v1[w], 0);
            row1[kp] = pair_half(v0[w], v1[w], 1);
        }
    }
}

template <int D>
struct RowBlock {
    u32x4_t qop[D / 32];   // Q^T operand: row l%16, dims kk*32 + lg*8 .. +7
    f32x4_t acc[D / 16];   // O^T: dims 16e + 4lg + i of row l%16
    float m, lsum;
    int pos;               // causal position of row l%16 (last visible key)
};

template <int D>
__device__ __forceinline__ void compute_tile(RowBlock<D> &rb, const Smem<D> &sm, int kv0,
                                             int L, bool masked, float scale_log2, int n,
                                             int lg)
{
    // S^T for the 4 key sub-tiles of 16
    f32x4_t s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const u32x4_t kop =
                *(const u32x4_t *)&sm.k[(16 * kt + n) * Smem<D>::kKStride + kk * 32 + lg * 8];
            s[kt] = mfma16x16x32(kop, rb.qop[kk], s[kt]);
        }
    }
    float x[16];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[4 * kt + i] = s[kt][i] * scale_log2;
    if (masked) {
        const int lim = min(rb.pos, L - 1);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kv0 + 16 * kt + 4 * lg + i > lim)
                    x[4 * kt + i] = kNegInf;
    }
    float bm = x[0];
#pragma unroll
    for (int j = 1; j < 16; ++j)
        bm = fmaxf(bm, x[j]);
    bm = group4_max(bm);
    // a row whose keys in this tile are all masked keeps its state (bm = -inf)
    const float m_new = (bm > rb.m + kRescaleSlack) ? bm : rb.m;
    if (__any(m_new != rb.m)) {
        const float alpha = exp2_fast(rb.m - m_new);
        rb.lsum *= alpha;
#pragma unroll
        for (int e = 0; e < D / 16; ++e)
            rb.acc[e] *= alpha;
        rb.m = m_new;
    }
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        p[j] = rb.m == kNegInf ? 0.f : exp2_fast(x[j] - rb.m);
        rb.lsum += p[j];
    }
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
        const u32x4_t pop = {pack_bf16(p[8 * ps + 0], p[8 * ps + 1]),
                             pack_bf16(p[8 * ps + 2], p[8 * ps + 3]),
                             pack_bf16(p[8 * ps + 4], p[8 * ps + 5]),
                             pack_bf16(p[8 * ps + 6], p[8 * ps + 7])};
#pragma unroll
        for (int e = 0; e < D / 16; ++e) {
            const uint16_t *vrow = &sm.vt[(16 * e + n) * Smem<D>::kVStride + 32 * ps + 4 * lg];
            const u32x2_t lo = *(const u32x2_t *)vrow;
            const u32x2_t hi = *(const u32x2_t *)(vrow + 16);
            const u32x4_t aop = {lo[0], lo[1], hi[0], hi[1]};
            rb.acc[e] = mfma16x16x32(aop, pop, rb.acc[e]);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_bf16(PrefillArgs a)
{
    const int qt = a.num_q_tiles - 1 - (int)blockIdx.x;  // heaviest tiles first
    const int h = blockIdx.y, b = blockIdx.z;
    const int q0 = a.cu_seqlens_q[b];
    const int q_len = a.cu_seqlens_q[b + 1] - q0;
    const int row0 = qt * kBM;
    if (row0 >= q_len)
        return;  // uniform over the workgroup
    const int L = a.seq_lens[b];
    const int g = h / a.group;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 15, lg = lane >> 4;
    const int shift = L - q_len;  // position of query row i is shift + i

    RowBlock<D> rb[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = row0 + 32 * wave + 16 * r + n;
        rb[r].pos = shift + row;
        rb[r].m = kNegInf;
        rb[r].lsum = 0.f;
#pragma unroll
        for (int e = 0; e < D / 16; ++e)
            rb[r].acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (row < q_len) {
            const uint16_t *qrow = a.q + ((size_t)(q0 + row) * a.num_q_heads + h) * D;
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                rb[r].qop[kk] = *(const u32x4_t *)(qrow + kk * 32 + lg * 8);
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                rb[r].qop[kk] = u32x4_t{0, 0, 0, 0};
        }
    }

    // keys needed by the workgroup and by this wave
    const int last_row = min(row0 + kBM, q_len) - 1;
    const int kv_end = min(shift + last_row + 1, L);
    const int wave_first = row0 + 32 * wave;
    const int wave_last = min(wave_first + 31, q_len - 1);
    const int wave_kv_end = wave_first < q_len ? min(shift + wave_last + 1, L) : 0;
    const int wave_pos_first = shift + wave_first;

    __shared__ Smem<D> sm;
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    for (int kv0 = 0; kv0 < kv_end; kv0 += kBN) {
        __syncthreads();
        load_tile<D>(sm, a, bt, kv0, L, g);
        __syncthreads();
        if (kv0 < wave_kv_end) {
            const bool masked = (kv0 + kBN - 1 > wave_pos_first) || (kv0 + kBN > L);
#pragma unroll
            for (int r = 0; r < 2; ++r)
                compute_tile<D>(rb[r], sm, kv0, L, masked, a.scale_log2, n, lg);
        }
    }

    const float sink2 = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = row0 + 32 * wave + 16 * r + n;
        const float lsum = group4_sum(rb[r].lsum);
        const float M = fmaxf(rb[r].m, sink2);
        float scale = 0.f;
        if (M != kNegInf) {
            const float f = rb[r].m == kNegInf ? 0.f : exp2_fast(rb[r].m - M);
            const float den = lsum * f + (sink2 == kNegInf ? 0.f : exp2_fast(sink2 - M));
            scale = den > 0.f ? f / den : 0.f;
        }
        if (row < q_len) {
            uint16_t *orow = a.out + ((size_t)(q0 + row) * a.num_q_heads + h) * D;
#pragma unroll
            for (int e = 0; e < D / 16; ++e) {
                const u32x2_t w = {pack_bf16(rb[r].acc[e][0] * scale, rb[r].acc[e][1] * scale),
                                   pack_bf16(rb[r].acc[e][2] * scale, rb[r].acc[e][3] * scale)};
                *(u32x2_t *)(orow + 16 * e + 4 * lg) = w;
            }
        }
    }
}

template <int D>
hipError_t launch_d(const PrefillLaunch &p)
{
    PrefillArgs a;
    a.q = (const uint16_t *)p.q;
    a.k_cache = (const uint16_t *)p.k_cache;
    a.v_cache = (const uint16_t *)p.v_cache;
    a.block_table = p.block_table;
    a.seq_lens = p.seq_lens;
    a.cu_seqlens_q = p.cu_seqlens_q;
    a.sinks = p.sinks;
    a.out = (uint16_t *)p.out;
    a.num_q_heads = p.num_q_heads;
    a.num_kv_heads = p.num_kv_heads;
    a.group = p.num_q_heads / p.num_kv_heads;
    a.max_pages = p.max_pages_per_seq;
    a.num_q_tiles = (p.max_q_len + kBM - 1) / kBM;
    a.scale_log2 = p.scale * kLog2e;
    dim3 grid(a.num_q_tiles, p.num_q_heads, p.num_seqs);
    hipLaunchKernelGGL(prefill_bf16<D>, grid, dim3(kThreads), 0, p.stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillLaunch &p)
{
    if (p.num_seqs == 0 || p.max_q_len == 0 || p.total_q == 0)
        return hipSuccess;
    return p.head_dim == 64 ? launch_d<64>(p) : launch_d<128>(p);
}

}  // namespace attn
