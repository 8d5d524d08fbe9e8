// Split-KV decode for paged GQA attention with per-head sinks (bf16, gfx950).
//
// Method ("GPT-OSS on day 0", section "Sink Attention"): attention for one
// query token is parallelised over heads and over the KV length; every part
// keeps a running maximum m and running sum, and the sink is counted once.
// Here the sink is folded into the final merge of the parts rather than into
// the first part, which is the same arithmetic (the merge rescales every part
// to a common maximum that includes the sink).
//
// Work decomposition:
//   grid (max_splits, Hkv, B), 4 waves per workgroup.  Workgroup (s, g, b)
//   owns tokens [s*C, min((s+1)*C, L_b)) of sequence b and KV head g, and all
//   G = Hq/Hkv query heads that read KV head g.  Wave w takes the w-th quarter
//   of that range in blocks of 32 tokens (two 16-token HND page slabs).
//
// Per 32-token block, on the matrix cores (16x16x32 bf16 MFMA):
//   S^T[16 tok x 16 heads] = K[16 tok x d] * Q^T[d x 16 heads]   (per slab)
//   O^T[16 dims x 16 heads] += V^T[16 dims x 32 tok] * P^T[32 tok x 16 heads]
// The S^T accumulator of lane l holds tokens 4*(l/16)+i of head l%16, which
// is exactly the P^T operand lane l must supply, so P never leaves registers.
// V rows are loaded straight from HBM (each lane group reads whole rows) and
// the V^T operand is formed with 16-bit pair packing; there is no LDS staging
// in the token loop.  Heads beyond G (when G < 16) carry a zero query and are
// discarded.
//
// The four waves then merge their (m, l, acc) through LDS into one partial per
// (split, head); decode_merge combines the partials of all splits and the
// sink: M = max(max_s m_s, sink), out = sum_s acc_s 2^(m_s - M) /
// (sum_s l_s 2^(m_s - M) + 2^(sink - M)), all in base-2 units.
#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

struct SplitArgs {
    const uint16_t *__restrict__ q;
    const uint16_t *__restrict__ k_cache;
    const uint16_t *__restrict__ v_cache;
    const int32_t *__restrict__ block_table;
    const int32_t *__restrict__ seq_lens;
    float *__restrict__ part_ml;
    float *__restrict__ part_acc;
    int num_q_heads, num_kv_heads, group;
    int max_pages, max_splits, split_tokens, wave_tokens;
    float scale_log2;
};

template <int D>
struct VRowT;
template <>
struct VRowT<64> {
    using type = u32x2_t;  // 4 bf16: dims 4n .. 4n+3
};
template <>
struct VRowT<128> {
    using type = u32x4_t;  // 8 bf16: dims 8n .. 8n+7
};

// Registers of one 32-token block: K operands of both slabs, and the V row
// chunks of the 8 tokens this lane feeds to the PV product.
template <int D>
struct Block {
    using VRow = typename VRowT<D>::type;
    u32x4_t k[2][D / 32];
    VRow v[8];
};

template <int D>
__device__ __forceinline__ void load_block(Block<D> &blk, const uint16_t *__restrict__ kc,
                                           const uint16_t *__restrict__ vc,
                                           const int32_t *__restrict__ bt, int t0, int t_end,
                                           int g, int num_kv_heads, int n, int lg)
{
    using VRow = typename VRowT<D>::type;
    constexpr size_t slab = 16 * D;
    const int page0 = bt[t0 >> 4];
    const size_t base0 = ((size_t)page0 * num_kv_heads + g) * slab;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        blk.k[0][kk] = *(const u32x4_t *)(kc + base0 + n * D + kk * 32 + lg * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        blk.v[i] = *(const VRow *)(vc + base0 + (4 * lg + i) * D + n * (D / 16));
    if (t0 + 16 < t_end) {
        const int page1 = bt[(t0 >> 4) + 1];
        const size_t base1 = ((size_t)page1 * num_kv_heads + g) * slab;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            blk.k[1][kk] = *(const u32x4_t *)(kc + base1 + n * D + kk * 32 + lg * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            blk.v[4 + i] = *(const VRow *)(vc + base1 + (4 * lg + i) * D + n * (D / 16));
    } else {
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            blk.k[1][kk] = u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            blk.v[4 + i] = VRow{};
    }
}

template <int D>
struct WaveState {
    float m;     // running reference maximum (base-2 units), shared by the 4 lanes of a head
    float lsum;  // this lane's share of the running sum
    f32x4_t acc[D / 16];
};

template <int D>
__device__ __forceinline__ void compute_block(WaveState<D> &st, Block<D> &blk,
                                              const u32x4_t (&qop)[D / 32], int t0, int t_end,
                                              float scale_log2, int lg)
{
    using VRow = typename VRowT<D>::type;
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        s0 = mfma16x16x32(blk.k[0][kk], qop[kk], s0);
        s1 = mfma16x16x32(blk.k[1][kk], qop[kk], s1);
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = s0[i] * scale_log2;
        x[4 + i] = s1[i] * scale_log2;
    }
    if (t0 + 32 > t_end) {
        // tail block: mask scores and zero the V rows of tokens outside the
        // range (they may hold NaN, and 0 * NaN would poison every head)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (t0 + 4 * lg + i >= t_end) {
                x[i] = kNegInf;
                blk.v[i] = VRow{};
            }
            if (t0 + 16 + 4 * lg + i >= t_end) {
                x[4 + i] = kNegInf;
                blk.v[4 + i] = VRow{};
            }
        }
    }
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        bm = fmaxf(bm, x[i]);
    bm = group4_max(bm);
    const float m_new = (bm > st.m + kRescaleSlack) ? bm : st.m;
    if (__any(m_new != st.m)) {
        const float alpha = exp2_fast(st.m - m_new);  // 0 on the first block
        st.lsum *= alpha;
#pragma unroll
        for (int e = 0; e < D / 16; ++e)
            st.acc[e] *= alpha;
        st.m = m_new;
    }
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = exp2_fast(x[i] - st.m);
        st.lsum += p[i];
    }
    const u32x4_t pop = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                         pack_bf16(p[6], p[7])};
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
        const int w = e >> 1, sel = e & 1;
        const u32x4_t aop = {pair_half(blk.v[0][w], blk.v[1][w], sel),
                             pair_half(blk.v[2][w], blk.v[3][w], sel),
                             pair_half(blk.v[4][w], blk.v[5][w], sel),
                             pair_half(blk.v[6][w], blk.v[7][w], sel)};
        st.acc[e] = mfma16x16x32(aop, pop, st.acc[e]);
    }
}

template <int D>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_split_bf16(SplitArgs a)
{
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = a.seq_lens[b];
    const int wg_start = s * a.split_tokens;
    if (wg_start >= L)
        return;  // uniform over the workgroup, before any barrier
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 15, lg = lane >> 4;
    const int wg_end = min(wg_start + a.split_tokens, L);
    const int t_begin = wg_start + wave * a.wave_tokens;
    const int t_end = min(t_begin + a.wave_tokens, wg_end);

    // Q^T operand: column n = query head g*G + n, dims kk*32 + lg*8 .. +7
    u32x4_t qop[D / 32];
    const int h = g * a.group + n;
    if (n < a.group) {
        const uint16_t *qrow = a.q + ((size_t)b * a.num_q_heads + h) * D;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            qop[kk] = *(const u32x4_t *)(qrow + kk * 32 + lg * 8);
    } else {
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            qop[kk] = u32x4_t{0, 0, 0, 0};
    }

    WaveState<D> st;
    st.m = kNegInf;
    st.lsum = 0.f;
#pragma unroll
    for (int e = 0; e < D / 16; ++e)
        st.acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    const int nblocks = t_end > t_begin ? (t_end - t_begin + 31) >> 5 : 0;
    Block<D> bufA, bufB;
    if (nblocks > 0)
        load_block<D>(bufA, a.k_cache, a.v_cache, bt, t_begin, t_end, g, a.num_kv_heads, n, lg);
    for (int ib = 0; ib < nblocks; ib += 2) {
        const int t0 = t_begin + 32 * ib;
        if (ib + 1 < nblocks)
            load_block<D>(bufB, a.k_cache, a.v_cache, bt, t0 + 32, t_end, g, a.num_kv_heads, n,
                          lg);
        compute_block<D>(st, bufA, qop, t0, t_end, a.scale_log2, lg);
        if (ib + 1 >= nblocks)
            break;
        if (ib + 2 < nblocks)
            load_block<D>(bufA, a.k_cache, a.v_cache, bt, t0 + 64, t_end, g, a.num_kv_heads, n,
                          lg);
        compute_block<D>(st, bufB, qop, t0 + 32, t_end, a.scale_log2, lg);
    }
    const float lsum = group4_sum(st.lsum);

    // merge the waves' partial results through LDS
    constexpr int kStride = D + 1;  // padding spreads the 16 heads over banks
    __shared__ float s_m[kDecodeWaves][16];
    __shared__ float s_l[kDecodeWaves][16];
    __shared__ float s_acc[kDecodeWaves][16 * kStride];
    if (lg == 0) {
        s_m[wave][n] = st.m;
        s_l[wave][n] = lsum;
    }
#pragma unroll
    for (int e = 0; e < D / 16; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s_acc[wave][n * kStride + (D / 16) * (4 * lg + i) + e] = st.acc[e][i];
    __syncthreads();

    const size_t part_row = ((size_t)b * a.max_splits + s) * a.num_q_heads + (size_t)g * a.group;
    for (int idx = threadIdx.x; idx < a.group * D; idx += 64 * kDecodeWaves) {
        const int hn = idx / D, d = idx - hn * D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w)
            M = fmaxf(M, s_m[w][hn]);
        float acc = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
            const float mw = s_m[w][hn];
            const float f = mw == kNegInf ? 0.f : exp2_fast(mw - M);
            acc += f * s_acc[w][hn * kStride + d];
            l += f * s_l[w][hn];
        }
        a.part_acc[(part_row + hn) * D + d] = acc;
        if (d == 0) {
            a.part_ml[(part_row + hn) * 2 + 0] = M;
            a.part_ml[(part_row + hn) * 2 + 1] = l;
        }
    }
}

struct MergeArgs {
    const float *__restrict__ part_ml;
    const float *__restrict__ part_acc;
    const int32_t *__restrict__ seq_lens;
    const float *__restrict__ sinks;
    void *__restrict__ out;
    int num_q_heads, max_splits, split_tokens;
};

// One wave per (query head, sequence): combine the splits and fold the sink.
template <int D, bool kBf16Out>
__global__ __launch_bounds__(64) void decode_merge(MergeArgs a)
{
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int L = a.seq_lens[b];
    const int ns = (L + a.split_tokens - 1) / a.split_tokens;
    const float sink2 = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
    const size_t row0 = (size_t)b * a.max_splits * a.num_q_heads + h;
    const size_t sstride = a.num_q_heads;

    float M = sink2;
    for (int s = lane; s < ns; s += 64)
        M = fmaxf(M, a.part_ml[(row0 + s * sstride) * 2]);
    M = wave_max(M);

    constexpr int kPer = D / 64;
    float acc[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        acc[j] = 0.f;
    float den = 0.f;
    if (M != kNegInf) {
        den = sink2 == kNegInf ? 0.f : exp2_fast(sink2 - M);
        for (int s = 0; s < ns; ++s) {
            const size_t r = row0 + s * sstride;
            const float ms = a.part_ml[r * 2];
            const float f = ms == kNegInf ? 0.f : exp2_fast(ms - M);
            den += f * a.part_ml[r * 2 + 1];
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                acc[j] += f * a.part_acc[r * D + lane + 64 * j];
        }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const size_t o = ((size_t)b * a.num_q_heads + h) * D;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const float v = acc[j] * inv;
        if (kBf16Out)
            ((__bf16 *)a.out)[o + lane + 64 * j] = (__bf16)v;
        else
            ((float *)a.out)[o + lane + 64 * j] = v;
    }
}

template <int D>
hipError_t launch_split_d(const DecodeLaunch &p)
{
    SplitArgs a;
    a.q = (const uint16_t *)p.q;
    a.k_cache = (const uint16_t *)p.k_cache;
    a.v_cache = (const uint16_t *)p.v_cache;
    a.block_table = p.block_table;
    a.seq_lens = p.seq_lens;
    a.part_ml = p.part_ml;
    a.part_acc = p.part_acc;
    a.num_q_heads = p.num_q_heads;
    a.num_kv_heads = p.num_kv_heads;
    a.group = p.num_q_heads / p.num_kv_heads;
    a.max_pages = p.max_pages_per_seq;
    a.max_splits = p.max_splits;
    a.split_tokens = p.split_tokens;
    a.wave_tokens = p.split_tokens / kDecodeWaves;
    a.scale_log2 = p.scale * kLog2e;
    dim3 grid(p.max_splits, p.num_kv_heads, p.num_seqs);
    hipLaunchKernelGGL(decode_split_bf16<D>, grid, dim3(64 * kDecodeWaves), 0, p.stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_merge_d(const DecodeLaunch &p)
{
    MergeArgs m;
    m.part_ml = p.part_ml;
    m.part_acc = p.part_acc;
    m.seq_lens = p.seq_lens;
    m.sinks = p.sinks;
    m.out = p.out;
    m.num_q_heads = p.num_q_heads;
    m.max_splits = p.max_splits;
    m.split_tokens = p.split_tokens;
    const dim3 grid(p.num_q_heads, p.num_seqs);
    if (p.dtype == 1)
        hipLaunchKernelGGL((decode_merge<D, true>), grid, dim3(64), 0, p.stream, m);
    else
        hipLaunchKernelGGL((decode_merge<D, false>), grid, dim3(64), 0, p.stream, m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split_bf16(const DecodeLaunch &p)
{
    if (p.num_seqs == 0 || p.max_splits == 0)
        return hipSuccess;
    return p.head_dim == 64 ? launch_split_d<64>(p) : launch_split_d<128>(p);
}

hipError_t launch_decode_merge(const DecodeLaunch &p)
{
    if (p.num_seqs == 0)
        return hipSuccess;
    return p.head_dim == 64 ? launch_merge_d<64>(p) : launch_merge_d<128>(p);
}

}  // namespace attn
