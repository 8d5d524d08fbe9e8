// The split pass of the paged decode as device code that more than one kernel
// runs: decode_split_bf16 (decode.hip) and the one-launch mixed batch
// (prefill.hip), whose first workgroups take the split pass of its decode
// rows.  Method, work decomposition and per-block arithmetic are described at
// the top of decode.hip.  The names live in attn::split so that a file with
// kernels of its own (the prefill) can include them.
#pragma once
#include "common.h"
#include "kernels.h"

namespace attn {
namespace split {
namespace {

struct SplitArgs {
    const uint16_t *__restrict__ q;
    const uint16_t *__restrict__ k_cache;
    const uint16_t *__restrict__ v_cache;
    const int32_t *__restrict__ block_table;
    const int32_t *__restrict__ seq_lens;
    float *__restrict__ part_ml;   // [slots][G][2]
    float *__restrict__ part_acc;  // [slots][G][D]
    int num_seqs, num_q_heads, num_kv_heads, group, max_pages;
    int num_wgs;        // workgroups per head group
    int heads_per_wg;   // KV heads (waves) per workgroup
    int window;         // sliding window W (0: none)
    const int32_t *__restrict__ cu_seqlens_q;  // multi-token decode: [B + 1]; NULL: one token
    int q_max;          // query rows per sequence in the partial results (1 for decode)
    float scale_log2;
    const float *__restrict__ sinks;  // direct decode: per-head sink logits, or NULL
    uint16_t *__restrict__ out;       // direct decode: bf16 [B][Hq][D]
};

constexpr int kUnitTokens = 32;

// Oldest key a decode token at position L - 1 sees: 0, or L - W under a
// sliding window of W ("GPT OSS" model notes, section 4.1: even layers attend
// within a local window; section 11: the window is passed per call).
__device__ __forceinline__ int oldest_key(int L, int window)
{
    return (window > 0 && L > window) ? L - window : 0;
}

// The units of a sequence are the 32-token blocks from the one holding its
// oldest visible key to its last: units_of of them, the first being block
// first_unit.
__device__ __forceinline__ int first_unit(int L, int window)
{
    return oldest_key(L, window) / kUnitTokens;
}
__device__ __forceinline__ long long units_of(int L, int window)
{
    return (L + kUnitTokens - 1) / kUnitTokens - first_unit(L, window);
}

// First unit of workgroup w, and the workgroup that processes unit u (the
// largest w whose first unit is <= u).
__device__ __forceinline__ long long wave_first_unit(long long w, long long U, int nw)
{
    return w * U / nw;
}
__device__ __forceinline__ int wave_of_unit(long long u, long long U, int nw)
{
    return (int)(((u + 1) * nw - 1) / U);
}

// Wave-wide scan over the sequences.  Returns U, the total unit count; when
// `target` >= 0 also returns the sequence that holds unit `target` and the
// index of that sequence's first unit.
__device__ long long scan_units(const int32_t *__restrict__ seq_lens, int num_seqs, int window,
                                int lane, long long target, int *b_out, long long *base_out)
{
    long long carry = 0;
    bool found = false;
    for (int b0 = 0; b0 < num_seqs; b0 += 64) {
        const int b = b0 + lane;
        const long long nb = b < num_seqs ? units_of(seq_lens[b], window) : 0;
        long long incl = nb;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const long long y = __shfl_up(incl, off, 64);
            if (lane >= off)
                incl += y;
        }
        if (target >= 0 && !found) {
            const unsigned long long hit = __ballot(carry + incl > target);
            if (hit) {
                const int first = __builtin_ctzll(hit);
                *b_out = b0 + first;
                *base_out = carry + __shfl(incl - nb, first, 64);
                found = true;
            }
        }
        carry += __shfl(incl, 63, 64);
    }
    return carry;
}

// Values the wave agrees on but the compiler cannot prove uniform (they come
// out of shuffles and ballots): moving them to scalar registers turns the
// page-table and length reads into scalar loads, which are counted apart from
// the vector loads in flight, so prefetched K/V blocks are not waited for.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform64(long long v)
{
    const unsigned long long u = (unsigned long long)v;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// Read-only int32 data (page table, lengths) at a wave-uniform index, through
// the constant address space: the compiler may then use the scalar unit's
// load path, which it only does for memory it knows is not written while the
// kernel runs -- true of every input here.
__device__ __forceinline__ int load_scalar(const int32_t *p, long long idx)
{
    return ((const __attribute__((address_space(4))) int32_t *)p)[idx];
}

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

// Registers of one 32-token block: K of both slabs as loaded (coalesced:
// chunk j*64 + lane of a slab, 16 B each), and the V row chunks of the 8
// tokens this lane feeds to the PV product.
template <int D>
struct Block {
    using VRow = typename VRowT<D>::type;
    u32x4_t k[2][D / 32];
    VRow v[8];
};

// K slabs are read with whole rows per lane quad (consecutive lanes read
// consecutive 16-byte chunks) and with the non-temporal hint, the form the
// memory pipeline serves fastest, then moved through a per-wave LDS buffer
// into the MFMA operand layout (lane n reads row n).  Chunk cc of row r is
// stored at position cc ^ swz(r), which makes both the row writes and the
// column-of-rows reads free of LDS bank conflicts.
template <int D>
__device__ __forceinline__ int k_swizzle(int r)
{
    return D == 64 ? ((r >> 1) & 7) : (r & 15);
}

// Load one 32-token block starting at token t0.  kFull: both slabs lie inside
// the range (no branch, so the compiler can keep several blocks in flight).
// Otherwise a slab is loaded only when it holds a token of [t_lo, t_end):
// the second only when t0 + 16 < t_end, and the first only when t0 + 16 >
// t_lo (under a sliding window the block that holds the oldest visible key
// may begin with a whole page below the window, whose table entry is then
// never read).  Slabs not loaded are zero.
template <int D, bool kFull>
__device__ __forceinline__ void load_block(Block<D> &blk, const uint16_t *__restrict__ kc,
                                           const uint16_t *__restrict__ vc,
                                           const int32_t *__restrict__ bt, int t0, int t_end,
                                           int g, int num_kv_heads, int n, int lg, int t_lo = 0)
{
    using VRow = typename VRowT<D>::type;
    constexpr size_t slab = 16 * D;
    const int lane = lg * 16 + n;
    const int pg = uniform(t0 >> 4);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const bool live = kFull || (s == 0 ? t0 + 16 > t_lo : t0 + 16 < t_end);
        if (live) {
            const int page = load_scalar(bt, pg + s);
            const size_t base = ((size_t)page * num_kv_heads + g) * slab;
#pragma unroll
            for (int j = 0; j < D / 32; ++j)
                blk.k[s][j] = __builtin_nontemporal_load(
                    (const u32x4_t *)(kc + base + (j * 64 + lane) * 8));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                blk.v[4 * s + i] = __builtin_nontemporal_load(
                    (const VRow *)(vc + base + (4 * lg + i) * D + n * (D / 16)));
        } else {
#pragma unroll
            for (int j = 0; j < D / 32; ++j)
                blk.k[s][j] = u32x4_t{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                blk.v[4 * s + i] = VRow{};
        }
    }
}

// Query rows of one KV head, packed GQA-style into the 16 columns of the
// matrix instructions: column block cb, column n holds packed row
// r = 16 cb + n, i.e. query token r / G of the sequence's new tokens and
// query head g G + r % G.  Plain decode (one token) uses one block whose
// columns past G are idle; a multi-token decode (Lq tokens per sequence, as
// speculative or MTP drafts are verified) uses ceil(G Lq / 16) blocks, which
// share every K and V operand.
template <int D, int NCB>
struct WaveState {
    float m[NCB];     // running reference maximum (base-2 units), per column
    float lsum[NCB];  // this lane's share of its column's running sum
    f32x4_t acc[NCB][D / 16];
};

template <int D, int NCB, bool kMasked>
__device__ __forceinline__ void compute_block(WaveState<D, NCB> &st, Block<D> &blk,
                                              const u32x4_t (&qop)[NCB][D / 32], int t0,
                                              int t_lo, int t_end, const int (&col_end)[NCB],
                                              float scale_log2, int lg, u32x4_t *klds)
{
    using VRow = typename VRowT<D>::type;
    constexpr int kChunks = D / 8;  // 16-byte chunks per K row
    const int n = threadIdx.x & 15, lane = threadIdx.x & 63;
    // K rows -> LDS (swizzled), then the operand layout back: lane n, row n.
    // The exchange stays within the wave, whose LDS operations the hardware
    // performs in order; the wave barriers keep the compiler from moving the
    // reads above the writes, or the next block's writes above these reads.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < D / 32; ++j) {
            const int c = j * 64 + lane, r = c / kChunks, cc = c % kChunks;
            klds[(s * 16 + r) * kChunks + (cc ^ k_swizzle<D>(r))] = blk.k[s][j];
        }
    __builtin_amdgcn_wave_barrier();
    u32x4_t kop[2][D / 32];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            kop[s][kk] = klds[(s * 16 + n) * kChunks + ((kk * 4 + lg) ^ k_swizzle<D>(n))];
    if (kMasked) {
        // first or last block of a piece: zero the V rows of tokens outside
        // [t_lo, t_end) (past the end they may hold NaN, and 0 * NaN would
        // poison every column)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ta = t0 + 4 * lg + i, tb = ta + 16;
            if (ta >= t_end || ta < t_lo)
                blk.v[i] = VRow{};
            if (tb >= t_end || tb < t_lo)
                blk.v[4 + i] = VRow{};
        }
    }
    u32x4_t pop[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            s0 = mfma16x16x32(kop[0][kk], qop[cb][kk], s0);
            s1 = mfma16x16x32(kop[1][kk], qop[cb][kk], s1);
        }
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = s0[i] * scale_log2;
            x[4 + i] = s1[i] * scale_log2;
        }
        if (kMasked) {
            // tokens outside [t_lo, min(t_end, col_end)) are invisible to this
            // column's row; the block holds at least one visible token of
            // every row that has any key at all
            const int te = min(t_end, col_end[cb]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ta = t0 + 4 * lg + i, tb = ta + 16;
                if (ta >= te || ta < t_lo)
                    x[i] = kNegInf;
                if (tb >= te || tb < t_lo)
                    x[4 + i] = kNegInf;
            }
        }
        float bm = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i)
            bm = fmaxf(bm, x[i]);
        bm = group4_max(bm);
        const float m_new = (bm > st.m[cb] + kRescaleSlack) ? bm : st.m[cb];
        if (__any(m_new != st.m[cb])) {
            // 0 on a column's first visible block; 1 on columns the branch
            // does not concern (their rows may still have seen no key: then
            // both maxima are -inf)
            const float alpha = m_new == st.m[cb] ? 1.f : exp2_fast(st.m[cb] - m_new);
            st.lsum[cb] *= alpha;
#pragma unroll
            for (int e = 0; e < D / 16; ++e)
                st.acc[cb][e] *= alpha;
            st.m[cb] = m_new;
        }
        // a column whose row has seen no key yet keeps m = -inf: weights 0
        const float m_ref = st.m[cb] == kNegInf ? 0.f : st.m[cb];
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = exp2_fast(x[i] - m_ref);
            st.lsum[cb] += p[i];
        }
        pop[cb] = u32x4_t{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                          pack_bf16(p[6], p[7])};
    }
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
        const int w = e >> 1, sel = e & 1;
        const u32x4_t aop = {pair_half(blk.v[0][w], blk.v[1][w], sel),
                             pair_half(blk.v[2][w], blk.v[3][w], sel),
                             pair_half(blk.v[4][w], blk.v[5][w], sel),
                             pair_half(blk.v[6][w], blk.v[7][w], sel)};
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            st.acc[cb][e] = mfma16x16x32(aop, pop[cb], st.acc[cb][e]);
    }
}

// A sequence's whole result for one KV head and one query token: fold the
// sink into the normalisation (as decode_merge does with a single piece) and
// write the bf16 output rows.  Lane (n, lg) holds dims (D/16)(4 lg + i) + e
// of query head g G + n, i.e. D/4 consecutive dims.
template <int D>
__device__ __forceinline__ void store_final(const SplitArgs &a, const WaveState<D, 1> &st, int q_row,
                                            int g, int n, int lg)
{
    const float lsum = group4_sum(st.lsum[0]);
    if (n >= a.group)
        return;
    const int h = g * a.group + n;
    const float m = st.m[0];
    const float sink2 = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
    const float M = fmaxf(m, sink2);
    float scale = 0.f;
    if (M != kNegInf) {
        const float f = m == kNegInf ? 0.f : exp2_fast(m - M);
        const float den = lsum * f + (sink2 == kNegInf ? 0.f : exp2_fast(sink2 - M));
        scale = den > 0.f ? f / den : 0.f;
    }
    uint16_t *dst = a.out + ((size_t)q_row * a.num_q_heads + h) * D + (D / 4) * lg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t w[D / 32];
#pragma unroll
        for (int e = 0; e < D / 16; e += 2)
            w[e / 2] = pack_bf16(st.acc[0][e][i] * scale, st.acc[0][e + 1][i] * scale);
        if constexpr (D == 64)
            *(u32x2_t *)(dst + (D / 16) * i) = u32x2_t{w[0], w[1]};
        else
            *(u32x4_t *)(dst + (D / 16) * i) = u32x4_t{w[0], w[1], w[2], w[3]};
    }
}

// One piece: the tokens of [t_begin, t_end) (t_begin a multiple of 32) from
// t_lo on, of segment (b, g); the result goes to `slot`, or, when kFinal (the
// piece is the whole sequence, one query token), straight to the output.
// q_first / q_len: the sequence's query rows (q_len new tokens, the last
// ones of its L keys); the wave takes the packed rows row0 .. row0 + 16 NCB - 1.
template <int D, int NCB, bool kFinal = false>
__device__ __forceinline__ void run_piece(const SplitArgs &a, int row0, int b, int g, int t_begin,
                                          int t_lo, int t_end, int L, int q_first, int q_len,
                                          long long slot, int n, int lg, u32x4_t *klds)
{
    b = uniform(b);
    g = uniform(g);
    t_begin = uniform(t_begin);
    t_lo = uniform(t_lo);
    t_end = uniform(t_end);
    L = uniform(L);
    q_first = uniform(q_first);
    q_len = uniform(q_len);
    // Q^T operands: column n of block cb = packed row 16 cb + n (query token
    // tok = row / G, head g G + row % G), dims kk*32 + lg*8 .. +7; rows of
    // no token are zero and never stored.  col_end: one past the row's last
    // visible key (bottom-right causal among the new tokens).
    u32x4_t qop[NCB][D / 32];
    int col_end[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int row = row0 + 16 * cb + n, tok = row / a.group;
        col_end[cb] = L - q_len + tok + 1;
        if (tok < q_len) {
            const uint16_t *qrow =
                a.q + ((size_t)(q_first + tok) * a.num_q_heads + g * a.group + row % a.group) * D;
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                qop[cb][kk] = *(const u32x4_t *)(qrow + kk * 32 + lg * 8);
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                qop[cb][kk] = u32x4_t{0, 0, 0, 0};
        }
    }
    WaveState<D, NCB> st;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        st.m[cb] = kNegInf;
        st.lsum[cb] = 0.f;
#pragma unroll
        for (int e = 0; e < D / 16; ++e)
            st.acc[cb][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    // The block that holds the oldest key of a sliding window: loaded and
    // computed first.  At d = 64 with one column block it is computed only
    // after the ring below has issued its first loads, so that its round trip
    // overlaps theirs instead of preceding them (the order of the arithmetic,
    // and so the result, is unchanged); elsewhere the registers it would hold
    // meanwhile are not there to spare.
    constexpr bool kHeadLate = D == 64 && NCB == 1;
    const bool has_head = t_begin < t_lo;
    const int t_head = t_begin;
    Block<D> head;
    auto run_head = [&]() {
        if (has_head)
            compute_block<D, NCB, true>(st, head, qop, t_head, t_lo, t_end, col_end,
                                        a.scale_log2, lg, klds);
    };
    if (has_head) {
        load_block<D, false>(head, a.k_cache, a.v_cache, bt, t_head, t_end, g, a.num_kv_heads,
                             n, lg, t_lo);
        t_begin += kUnitTokens;
        if constexpr (!kHeadLate)
            run_head();
    }
    // Full blocks (keys every row sees) stream through a ring of register
    // buffers with loads issued ahead of the matrix work (two blocks ahead at
    // d = 64, one at d = 128, where a block is 16 KiB per wave, and one when
    // the packed query rows need the registers).  Prefetches
    // past the last full block re-read that block (a cache hit), so the loop
    // body has no branches around loads.  The rest -- a partial last block,
    // and the blocks with keys some new token may not see -- comes after.
    const int t_all = min(t_end, L - q_len + 1);  // keys below it: seen by every row
    const int nfull = t_all > t_begin ? (t_all - t_begin) / kUnitTokens : 0;
    const int t_last = t_begin + kUnitTokens * (nfull - 1);
    auto at = [&](int ib) { return min(t_begin + kUnitTokens * ib, t_last); };
    if (nfull > 0) {
        if constexpr (D == 64 && NCB < 4) {
            Block<D> b0, b1, b2;
            load_block<D, true>(b0, a.k_cache, a.v_cache, bt, at(0), t_end, g, a.num_kv_heads, n,
                                lg);
            load_block<D, true>(b1, a.k_cache, a.v_cache, bt, at(1), t_end, g, a.num_kv_heads, n,
                                lg);
            if constexpr (kHeadLate)
                run_head();
            for (int ib = 0; ib < nfull; ib += 3) {
                const int t0 = t_begin + kUnitTokens * ib;
                load_block<D, true>(b2, a.k_cache, a.v_cache, bt, at(ib + 2), t_end, g,
                                    a.num_kv_heads, n, lg);
                compute_block<D, NCB, false>(st, b0, qop, t0, t_lo, t_end, col_end,
                                             a.scale_log2, lg, klds);
                if (ib + 1 >= nfull)
                    break;
                load_block<D, true>(b0, a.k_cache, a.v_cache, bt, at(ib + 3), t_end, g,
                                    a.num_kv_heads, n, lg);
                compute_block<D, NCB, false>(st, b1, qop, t0 + 32, t_lo, t_end, col_end,
                                             a.scale_log2, lg, klds);
                if (ib + 2 >= nfull)
                    break;
                load_block<D, true>(b1, a.k_cache, a.v_cache, bt, at(ib + 4), t_end, g,
                                    a.num_kv_heads, n, lg);
                compute_block<D, NCB, false>(st, b2, qop, t0 + 64, t_lo, t_end, col_end,
                                             a.scale_log2, lg, klds);
            }
        } else if constexpr (D == 128 && NCB > 1) {
            // two column blocks of packed rows leave no registers for a
            // second block: one block at a time (the many waves of the
            // layers keep the memory busy)
            for (int ib = 0; ib < nfull; ++ib) {
                Block<D> b0;
                load_block<D, true>(b0, a.k_cache, a.v_cache, bt, at(ib), t_end, g,
                                    a.num_kv_heads, n, lg);
                compute_block<D, NCB, false>(st, b0, qop, t_begin + kUnitTokens * ib, t_lo,
                                             t_end, col_end, a.scale_log2, lg, klds);
            }
        } else {
            Block<D> b0, b1;
            load_block<D, true>(b0, a.k_cache, a.v_cache, bt, at(0), t_end, g, a.num_kv_heads, n,
                                lg);
            for (int ib = 0; ib < nfull; ib += 2) {
                const int t0 = t_begin + kUnitTokens * ib;
                load_block<D, true>(b1, a.k_cache, a.v_cache, bt, at(ib + 1), t_end, g,
                                    a.num_kv_heads, n, lg);
                compute_block<D, NCB, false>(st, b0, qop, t0, t_lo, t_end, col_end,
                                             a.scale_log2, lg, klds);
                if (ib + 1 >= nfull)
                    break;
                load_block<D, true>(b0, a.k_cache, a.v_cache, bt, at(ib + 2), t_end, g,
                                    a.num_kv_heads, n, lg);
                compute_block<D, NCB, false>(st, b1, qop, t0 + 32, t_lo, t_end, col_end,
                                             a.scale_log2, lg, klds);
            }
        }
    } else if constexpr (kHeadLate) {
        run_head();
    }
    for (int t0 = t_begin + kUnitTokens * nfull; t0 < t_end; t0 += kUnitTokens) {
        Block<D> bt_tail;
        load_block<D, false>(bt_tail, a.k_cache, a.v_cache, bt, t0, t_end, g, a.num_kv_heads, n,
                             lg);
        compute_block<D, NCB, true>(st, bt_tail, qop, t0, t_lo, t_end, col_end, a.scale_log2,
                                    lg, klds);
    }
    if constexpr (kFinal) {
        static_assert(NCB == 1, "one query token");
        store_final<D>(a, st, q_first, g, n, lg);
        return;
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const float lsum = group4_sum(st.lsum[cb]);
        const int row = row0 + 16 * cb + n, tok = row / a.group;
        if (tok < q_len) {
            // partial-result row: (slot, query token, query head)
            const size_t prow = ((size_t)slot * a.q_max + tok) * a.num_q_heads +
                                (size_t)g * a.group + row % a.group;
            if (lg == 0)
                *(float2 *)(a.part_ml + prow * 2) = make_float2(st.m[cb], lsum);
            // lane (n, lg) holds dims (D/16)*(4*lg + i) + e of its row
            float *dst = a.part_acc + prow * D;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e4 = 0; e4 < D / 16; e4 += 4)
                    *(f32x4_t *)(dst + (D / 16) * (4 * lg + i) + e4) =
                        f32x4_t{st.acc[cb][e4][i], st.acc[cb][e4 + 1][i],
                                st.acc[cb][e4 + 2][i], st.acc[cb][e4 + 3][i]};
        }
    }
}

// Where a split workgroup finds its place: x() is its workgroup index within
// its KV-head group, y() the group, z() the grid layer of packed query rows.
// GridIdx: decode_split_bf16's own 3-D grid.  FlatIdx: a 1-D grid whose first
// workgroups are split workgroups, wx of them per KV-head group, one layer.
struct GridIdx {
    __device__ unsigned x() const { return blockIdx.x; }
    __device__ unsigned y() const { return blockIdx.y; }
    __device__ unsigned z() const { return blockIdx.z; }
};
struct FlatIdx {
    unsigned wx;
    __device__ unsigned x() const { return blockIdx.x % wx; }
    __device__ unsigned y() const { return blockIdx.x / wx; }
    __device__ unsigned z() const { return 0u; }
};

// The split pass of one workgroup (placed by idx): every piece of its unit
// range, partial results to their slots.  The waves are independent (no
// barrier): a wave whose KV head lies past the last one returns at once.
template <int D, int NCB, class Idx>
__device__ __forceinline__ void split_body(const SplitArgs &a, const Idx &idx)
{
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, lg = lane >> 4;
    const int g = uniform(idx.y() * a.heads_per_wg + (threadIdx.x >> 6));
    if (g >= a.num_kv_heads)
        return;  // the last head group may be partial (waves are independent)
    const int w = idx.x();
    const int row0 = 16 * NCB * idx.z();  // this layer's packed rows
    // per-wave K staging buffer: one 32-token block of K (dynamic LDS,
    // heads_per_wg * 64 * D bytes)
    extern __shared__ u32x4_t s_k[];
    u32x4_t *klds = s_k + (threadIdx.x >> 6) * (2 * 16 * (D / 8));
    int b = 0;
    long long base = 0;
    const long long U = scan_units(a.seq_lens, a.num_seqs, a.window, lane, -1, &b, &base);
    const long long u_begin = wave_first_unit(w, U, a.num_wgs);
    const long long u_end = wave_first_unit(w + 1, U, a.num_wgs);
    if (u_begin >= u_end)
        return;  // no unit for this workgroup
    scan_units(a.seq_lens, a.num_seqs, a.window, lane, u_begin, &b, &base);
    b = uniform(b);
    base = uniform64(base);
    long long u = uniform64(u_begin);
    const long long u_stop = uniform64(u_end);
    while (u < u_stop) {
        // sequence b holds units [base, base + nblk): its 32-token blocks
        // from block first_unit on
        const int L = load_scalar(a.seq_lens, b);
        const long long nblk = units_of(L, a.window);
        const int fu = first_unit(L, a.window);
        const long long piece_end = min(u_stop, base + nblk);
        const int t_begin = ((int)(u - base) + fu) * kUnitTokens;
        const int t_end = min(((int)(piece_end - base) + fu) * kUnitTokens, L);
        int q_first = b, q_len = 1;
        if (a.cu_seqlens_q) {
            q_first = load_scalar(a.cu_seqlens_q, b);
            q_len = load_scalar(a.cu_seqlens_q, b + 1) - q_first;
        }
        run_piece<D, NCB>(a, row0, b, g, t_begin, oldest_key(L, a.window), t_end, L, q_first, q_len,
                          (long long)b + w, n, lg, klds);
        u = piece_end;
        if (u < u_stop) {
            // next sequence with at least one unit
            base += nblk;
            do {
                ++b;
            } while (load_scalar(a.seq_lens, b) == 0);
        }
    }
}

// The split pass's arguments for a decode launch description.
inline SplitArgs split_args(const DecodeLaunch &p)
{
    SplitArgs a;
    a.q = (const uint16_t *)p.q;
    a.k_cache = (const uint16_t *)p.k_cache;
    a.v_cache = (const uint16_t *)p.v_cache;
    a.block_table = p.block_table;
    a.seq_lens = p.seq_lens;
    a.part_ml = p.part_ml;
    a.part_acc = p.part_acc;
    a.num_seqs = p.num_seqs;
    a.num_q_heads = p.num_q_heads;
    a.num_kv_heads = p.num_kv_heads;
    a.group = p.num_q_heads / p.num_kv_heads;
    a.max_pages = p.max_pages_per_seq;
    a.num_wgs = p.num_wgs;
    a.heads_per_wg = p.heads_per_wg;
    a.window = p.window;
    a.cu_seqlens_q = p.cu_seqlens_q;
    a.q_max = p.q_max;
    a.scale_log2 = p.scale * kLog2e;
    a.sinks = nullptr;
    a.out = nullptr;
    return a;
}

// Dynamic LDS of the split pass: one 32-token K block per wave.
template <int D>
constexpr size_t split_lds_bytes(int heads_per_wg)
{
    return (size_t)heads_per_wg * 2 * 16 * (D / 8) * sizeof(u32x4_t);
}

}  // namespace
}  // namespace split
}  // namespace attn
