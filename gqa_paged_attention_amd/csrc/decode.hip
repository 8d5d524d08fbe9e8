// Split-KV decode for paged GQA attention with per-head sinks (bf16, gfx950).
//
// Method ("GPT-OSS on day 0", section "Sink Attention"): attention for one
// query token is parallelised over heads and over the KV length; every part
// keeps a running maximum m and running sum, and the sink is counted once.
// Here the sink is folded into the final merge of the parts rather than into
// the first part, which is the same arithmetic (the merge rescales every part
// to a common maximum that includes the sink).
//
// Work decomposition (persistent, balanced):
//   A unit is one 32-token block (two 16-token HND pages) of one sequence b,
//   for all KV heads of a head group; units are numbered sequence-major, and
//   there are U = sum_b ceil(L_b / 32) of them.  A workgroup has one wave per
//   KV head of its group (up to 4), and workgroup w of a group takes units
//   [floor(w U / NWG), floor((w+1) U / NWG)).  Its waves walk the same token
//   range, so the slabs of all heads of a page -- contiguous in the HND
//   layout -- are requested together, and every workgroup streams the same
//   number of blocks to within one.  NWG is sized from host integers to fill
//   the chip once.  The part of sequence b covered by workgroup w is a
//   "piece"; its partial result goes to slot (b + w), which is unique,
//   depends only on the sequence lengths (never on page ids) and needs at
//   most (num_seqs + NWG) slots.
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
// Loads run ahead of the matrix work (see run_piece).  decode_merge then combines
// the pieces of each (sequence, head) in logical order together with the
// sink: M = max(max_p m_p, sink), out = sum_p acc_p 2^(m_p - M) /
// (sum_p l_p 2^(m_p - M) + 2^(sink - M)), all in base-2 units.
#include "common.h"
#include "kernels.h"
#include "split.h"

namespace attn {
namespace {

using namespace split;

template <int D, int NCB>
__global__ __launch_bounds__(512) void decode_split_bf16(SplitArgs a)
{
    split_body<D, NCB>(a, GridIdx{});
}

// Direct decode, for sliding windows short enough that one wave per
// (sequence, KV head) covers a sequence's visible keys quickly: no split, no
// partial results, no merge launch.  The wave runs the same block loop as a
// split piece over the blocks from the one holding the oldest visible key to
// the last, then folds the sink and writes the output.
template <int D>
__global__ __launch_bounds__(64) void decode_direct_bf16(SplitArgs a)
{
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, lg = lane >> 4;
    const int b = blockIdx.x, g = blockIdx.y;
    extern __shared__ u32x4_t s_k[];
    const int L = load_scalar(a.seq_lens, b);
    const int t_lo = oldest_key(L, a.window);
    run_piece<D, 1, true>(a, 0, b, g, first_unit(L, a.window) * kUnitTokens, t_lo, L, L, b, 1, 0, n,
                          lg, s_k);
}

struct MergeArgs {
    const float *__restrict__ part_ml;
    const float *__restrict__ part_acc;
    const int32_t *__restrict__ seq_lens;
    const float *__restrict__ sinks;
    void *__restrict__ out;
    int num_seqs, num_q_heads, num_kv_heads, num_wgs;
    int window;  // sliding window W (0: none); places the pieces as the split pass does
    const int32_t *__restrict__ cu_seqlens_q;  // multi-token decode: [B + 1]; NULL: one token
    int q_max;   // query rows per sequence in the partial results
};

// One workgroup per (sequence, KV head, query token), one wave per query
// head of the group: combine the pieces of the sequence in logical order and
// fold the sink.  The work is two dependent memory round trips: the sequence lengths
// (which place the sequence's pieces), then every piece's (m, l) -- one
// piece per lane -- together with the accumulators of up to kBatch pieces.
template <int D, bool kBf16Out>
__global__ __launch_bounds__(1024) void decode_merge(MergeArgs a)
{
    constexpr int kPer = D / 64;   // output dims per lane
    constexpr int kBatch = 4;      // pieces whose accumulators are loaded at once
    const int b = blockIdx.x, lane = threadIdx.x & 63, tok = blockIdx.z;
    int q_first = b, q_len = 1;
    if (a.cu_seqlens_q) {
        q_first = a.cu_seqlens_q[b];
        q_len = a.cu_seqlens_q[b + 1] - q_first;
    }
    if (tok >= q_len)
        return;  // uniform over the workgroup
    const int group = a.num_q_heads / a.num_kv_heads;
    const int h = blockIdx.y * group + (threadIdx.x >> 6);
    const float sink2 = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
    const int L = a.seq_lens[b];
    const long long nblk = units_of(L, a.window);

    int w_lo = 0, w_hi = -1;
    long long U = 0;
    if (nblk > 0) {
        // all units, and the units of the sequences before b, in one pass
        long long before = 0, total = 0;
        for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
            const int bi = b0 + lane;
            const long long u = bi < a.num_seqs ? units_of(a.seq_lens[bi], a.window) : 0;
            total += u;
            before += bi < b ? u : 0;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            total += __shfl_xor(total, off, 64);
            before += __shfl_xor(before, off, 64);
        }
        U = total;
        w_lo = wave_of_unit(before, U, a.num_wgs);
        w_hi = wave_of_unit(before + nblk - 1, U, a.num_wgs);
    }
    const int npieces = w_hi - w_lo + 1;
    // workgroups in [w_lo, w_hi] with an empty unit range (possible when
    // there are fewer units than workgroups) wrote nothing and are skipped
    auto live = [&](int w) {
        return wave_first_unit(w, U, a.num_wgs) < wave_first_unit(w + 1, U, a.num_wgs);
    };
    auto row_of = [&](int w) { return ((size_t)(b + w) * a.q_max + tok) * a.num_q_heads + h; };

    // (m, l) of piece w_lo + i + 64 k in lane i
    float M = sink2;
    float mp[2] = {kNegInf, kNegInf}, lp[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int w = w_lo + lane + 64 * k;
        if (w <= w_hi && live(w)) {
            const float2 ml = *(const float2 *)(a.part_ml + row_of(w) * 2);
            mp[k] = ml.x;
            lp[k] = ml.y;
        }
    }
    for (int w = w_lo + lane + 128; w <= w_hi; w += 64)  // more than 128 pieces: max only
        if (live(w))
            M = fmaxf(M, a.part_ml[row_of(w) * 2]);
    M = wave_max(fmaxf(M, fmaxf(mp[0], mp[1])));

    float acc[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        acc[k] = 0.f;
    float den = 0.f;
    if (M != kNegInf) {
        den = sink2 == kNegInf ? 0.f : exp2_fast(sink2 - M);
        for (int i0 = 0; i0 < npieces; i0 += kBatch) {
            float part[kBatch][kPer];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int w = w_lo + i0 + j;
                const bool ok = i0 + j < npieces;
#pragma unroll
                for (int k = 0; k < kPer; ++k)
                    part[j][k] = ok ? a.part_acc[row_of(w) * D + lane + 64 * k] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int i = i0 + j, w = w_lo + i;
                if (i >= npieces || !live(w))
                    continue;
                float m, l;
                if (i < 128) {
                    m = __shfl(i < 64 ? mp[0] : mp[1], i & 63, 64);
                    l = __shfl(i < 64 ? lp[0] : lp[1], i & 63, 64);
                } else {
                    m = a.part_ml[row_of(w) * 2];
                    l = a.part_ml[row_of(w) * 2 + 1];
                }
                const float f = m == kNegInf ? 0.f : exp2_fast(m - M);
                den += f * l;
#pragma unroll
                for (int k = 0; k < kPer; ++k)
                    acc[k] += f * part[j][k];
            }
        }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const size_t o = ((size_t)(q_first + tok) * a.num_q_heads + h) * D;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const float v = acc[k] * inv;
        if (kBf16Out)
            ((__bf16 *)a.out)[o + lane + 64 * k] = (__bf16)v;
        else
            ((float *)a.out)[o + lane + 64 * k] = v;
    }
}

// The merge with one wave per (sequence, KV head, query token), taking all G
// query heads of the group: fewer waves than decode_merge's one per head
// (the multi-token decode has G x tokens rows per KV head, which as single
// waves would not fit on the chip at once), in the same arithmetic and order
// (so the two give the same bits).  After the unit scan that places the
// sequence's pieces, the lanes take one piece each (64 at a time) for the
// common maximum of every head (sink included), keeping the (m_p, l_p) of the
// first 64 pieces; then, 32 pieces at a time, each piece's weight
// 2^(m_p - M) and sum l_p (from those registers, read again only past 64
// pieces) go to LDS, and every lane takes
// its (head, 4-dim chunk) items through the pieces in order: denominator from
// the sink term on plus f_p l_p, values f_p acc_p, kPB pieces' loads in
// flight at a time.  Workgroups without a unit wrote nothing; they count
// with weight 0 and are not read.
template <int D, bool kBf16Out>
__global__ __launch_bounds__(64) void decode_merge_group(MergeArgs a)
{
    constexpr int kMaxG = 16;
    constexpr int kChunks = D / 4;                // float4 chunks of a head's row
    constexpr int kItems = kMaxG * kChunks / 64;  // items per lane at G = 16
    constexpr int kPB = D == 64 ? 4 : 2;          // pieces whose loads are in flight together
    constexpr int kPiecesPerPass = 32;
    __shared__ float wf[kPiecesPerPass * kMaxG], wl[kPiecesPerPass * kMaxG];
    const int b = blockIdx.x, g = blockIdx.y, tok = blockIdx.z, lane = threadIdx.x;
    int q_first = b, q_len = 1;
    if (a.cu_seqlens_q) {
        q_first = a.cu_seqlens_q[b];
        q_len = a.cu_seqlens_q[b + 1] - q_first;
    }
    if (tok >= q_len)
        return;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int h0 = g * G;
    const int L = a.seq_lens[b];
    const long long nblk = units_of(L, a.window);
    int w_lo = 0, w_hi = -1;
    long long U = 0;
    if (nblk > 0) {
        long long before = 0, total = 0;
        for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
            const int bi = b0 + lane;
            const long long u = bi < a.num_seqs ? units_of(a.seq_lens[bi], a.window) : 0;
            total += u;
            before += bi < b ? u : 0;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            total += __shfl_xor(total, off, 64);
            before += __shfl_xor(before, off, 64);
        }
        U = total;
        w_lo = wave_of_unit(before, U, a.num_wgs);
        w_hi = wave_of_unit(before + nblk - 1, U, a.num_wgs);
    }
    auto live = [&](int w) {
        return wave_first_unit(w, U, a.num_wgs) < wave_first_unit(w + 1, U, a.num_wgs);
    };
    // partial-result row of piece w for the group's first head
    auto row = [&](int w) {
        return ((size_t)(b + w) * a.q_max + tok) * a.num_q_heads + h0;
    };

    // (m, l) of piece w_lo + lane (the first 64 pieces) stay in registers for
    // the weights below
    float M[kMaxG], m_own[kMaxG], l_own[kMaxG];
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
        M[hh] = (hh < G && a.sinks) ? a.sinks[h0 + hh] * kLog2e : kNegInf;
        m_own[hh] = kNegInf;
        l_own[hh] = 0.f;
    }
    for (int w0 = w_lo; w0 <= w_hi; w0 += 64) {
        const int w = w0 + lane;
        if (w <= w_hi && live(w)) {
            const float *ml = a.part_ml + row(w) * 2;
#pragma unroll
            for (int hh = 0; hh < kMaxG; ++hh)
                if (hh < G) {
                    const float2 v = *(const float2 *)(ml + 2 * hh);
                    M[hh] = fmaxf(M[hh], v.x);
                    if (w0 == w_lo) {
                        m_own[hh] = v.x;
                        l_own[hh] = v.y;
                    }
                }
        }
    }
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh)
        if (hh < G)
            M[hh] = wave_max(M[hh]);

    // this lane's items: head hi[k], chunk ci[k]; den from the sink term
    int hi[kItems], ci[kItems];
    float den[kItems];
    f32x4_t acc[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const int i = lane + 64 * k;
        hi[k] = i / kChunks;
        ci[k] = i % kChunks;
        acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        den[k] = 0.f;
    }
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
        if (hh < G) {
            const float sink2 = a.sinks ? a.sinks[h0 + hh] * kLog2e : kNegInf;
            const float d0 = sink2 == kNegInf ? 0.f : exp2_fast(sink2 - M[hh]);
#pragma unroll
            for (int k = 0; k < kItems; ++k)
                if (hi[k] == hh)
                    den[k] = d0;
        }
    }
    for (int w0 = w_lo; w0 <= w_hi; w0 += kPiecesPerPass) {
        const int w = w0 + lane;
        // the pass's pieces among the first 64 come from the lanes that hold them
        const int off = w0 - w_lo;
        const bool ok = lane < kPiecesPerPass && w <= w_hi && live(w);
#pragma unroll
        for (int hh = 0; hh < kMaxG; ++hh) {
            if (hh < G) {
                float mv = kNegInf, lv = 0.f;
                if (off < 64) {
                    mv = __shfl(m_own[hh], (off + lane) & 63, 64);
                    lv = __shfl(l_own[hh], (off + lane) & 63, 64);
                }
                if (lane < kPiecesPerPass) {
                    float f = 0.f, l = 0.f;
                    if (ok) {
                        if (off >= 64) {
                            const float2 ml = *(const float2 *)(a.part_ml + (row(w) + hh) * 2);
                            mv = ml.x;
                            lv = ml.y;
                        }
                        f = mv == kNegInf ? 0.f : exp2_fast(mv - M[hh]);
                        l = lv;
                    }
                    wf[lane * kMaxG + hh] = f;
                    wl[lane * kMaxG + hh] = l;
                }
            }
        }
        __syncthreads();
        const int cnt = min(kPiecesPerPass, w_hi - w0 + 1);
        for (int j0 = 0; j0 < cnt; j0 += kPB) {
            f32x4_t v[kItems][kPB];
            float fj[kItems][kPB], lj[kItems][kPB];
#pragma unroll
            for (int k = 0; k < kItems; ++k) {
                const bool item = hi[k] < G;
#pragma unroll
                for (int jj = 0; jj < kPB; ++jj) {
                    const int j = j0 + jj;
                    const bool in = item && j < cnt;
                    const float f = in ? wf[j * kMaxG + hi[k]] : 0.f;
                    fj[k][jj] = f;
                    lj[k][jj] = in ? wl[j * kMaxG + hi[k]] : 0.f;
                    v[k][jj] = f != 0.f ? *(const f32x4_t *)(a.part_acc +
                                                              (row(w0 + j) + hi[k]) * D +
                                                              4 * ci[k])
                                        : f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int k = 0; k < kItems; ++k)
#pragma unroll
                for (int jj = 0; jj < kPB; ++jj) {
                    den[k] += fj[k][jj] * lj[k][jj];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[k][e] += fj[k][jj] * v[k][jj][e];
                }
        }
        __syncthreads();
    }
    const size_t o = (size_t)(q_first + tok) * a.num_q_heads + h0;
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        if (hi[k] < G) {
            const float inv = den[k] > 0.f ? 1.f / den[k] : 0.f;
            const size_t e0 = (o + hi[k]) * D + 4 * ci[k];
            if constexpr (kBf16Out) {
                *(u32x2_t *)((uint16_t *)a.out + e0) =
                    u32x2_t{pack_bf16(acc[k][0] * inv, acc[k][1] * inv),
                            pack_bf16(acc[k][2] * inv, acc[k][3] * inv)};
            } else {
                *(f32x4_t *)((float *)a.out + e0) = acc[k] * inv;
            }
        }
    }
}

template <int D, int NCB>
hipError_t launch_split_d(const DecodeLaunch &p)
{
    const SplitArgs a = split_args(p);
    // row groups of 16 NCB packed rows each, one per grid layer
    const int rows = a.group * p.q_max;
    const unsigned groups = (unsigned)((rows + 16 * NCB - 1) / (16 * NCB));
    const dim3 grid(p.num_wgs, (p.num_kv_heads + p.heads_per_wg - 1) / p.heads_per_wg, groups);
    const size_t lds = split_lds_bytes<D>(p.heads_per_wg);
    hipLaunchKernelGGL((decode_split_bf16<D, NCB>), grid, dim3(64 * p.heads_per_wg), lds,
                       p.stream, a);
    return hipGetLastError();
}

// Column blocks of packed query rows, G * (query rows per sequence) of them:
// up to NCB blocks of 16 share each wave's K/V reads (NCB <= 4 at d = 64, 2 at
// d = 128, where more would not fit the registers); more rows take further
// grid layers, which read the K/V again.
template <int D>
hipError_t launch_split_rows(const DecodeLaunch &p)
{
    const int rows = (p.num_q_heads / p.num_kv_heads) * p.q_max;
    if (rows <= 16)
        return launch_split_d<D, 1>(p);
    if constexpr (D == 64) {
        if (rows <= 32)
            return launch_split_d<D, 2>(p);
        return launch_split_d<D, 4>(p);
    } else {
        return launch_split_d<D, 2>(p);
    }
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
    m.num_seqs = p.num_seqs;
    m.num_q_heads = p.num_q_heads;
    m.num_kv_heads = p.num_kv_heads;
    m.num_wgs = p.num_wgs;
    m.window = p.window;
    m.cu_seqlens_q = p.cu_seqlens_q;
    m.q_max = p.q_max;
    const dim3 grid(p.num_seqs, p.num_kv_heads, p.q_max);
    if (p.q_max > 1) {
        // multi-token decode: one wave per (sequence, KV head, token)
        if (p.dtype == 1)
            hipLaunchKernelGGL((decode_merge_group<D, true>), grid, dim3(64), 0, p.stream, m);
        else
            hipLaunchKernelGGL((decode_merge_group<D, false>), grid, dim3(64), 0, p.stream, m);
        return hipGetLastError();
    }
    const dim3 block(64 * (p.num_q_heads / p.num_kv_heads));
    if (p.dtype == 1)
        hipLaunchKernelGGL((decode_merge<D, true>), grid, block, 0, p.stream, m);
    else
        hipLaunchKernelGGL((decode_merge<D, false>), grid, block, 0, p.stream, m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split_bf16(const DecodeLaunch &p)
{
    if (p.num_seqs == 0 || p.num_wgs == 0)
        return hipSuccess;
    return p.head_dim == 64 ? launch_split_rows<64>(p) : launch_split_rows<128>(p);
}

hipError_t launch_decode_direct_bf16(const DecodeLaunch &p)
{
    if (p.num_seqs == 0)
        return hipSuccess;
    SplitArgs a = {};
    a.q = (const uint16_t *)p.q;
    a.k_cache = (const uint16_t *)p.k_cache;
    a.v_cache = (const uint16_t *)p.v_cache;
    a.block_table = p.block_table;
    a.seq_lens = p.seq_lens;
    a.num_seqs = p.num_seqs;
    a.num_q_heads = p.num_q_heads;
    a.num_kv_heads = p.num_kv_heads;
    a.group = p.num_q_heads / p.num_kv_heads;
    a.max_pages = p.max_pages_per_seq;
    a.window = p.window;
    a.q_max = 1;
    a.scale_log2 = p.scale * kLog2e;
    a.sinks = p.sinks;
    a.out = (uint16_t *)p.out;
    const dim3 grid(p.num_seqs, p.num_kv_heads);
    if (p.head_dim == 64)
        hipLaunchKernelGGL(decode_direct_bf16<64>, grid, dim3(64), 2 * 16 * (64 / 8) * 16,
                           p.stream, a);
    else
        hipLaunchKernelGGL(decode_direct_bf16<128>, grid, dim3(64), 2 * 16 * (128 / 8) * 16,
                           p.stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeLaunch &p)
{
    if (p.num_seqs == 0)
        return hipSuccess;
    return p.head_dim == 64 ? launch_merge_d<64>(p) : launch_merge_d<128>(p);
}

}  // namespace attn
