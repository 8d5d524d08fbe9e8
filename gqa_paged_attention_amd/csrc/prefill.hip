// Causal prefill for paged GQA attention with per-head sinks (bf16, gfx950).
//
// Each query row runs the online softmax of "GPT-OSS on day 0" (section
// "Sink Attention": running maximum and sum over blocks of keys) and the sink
// is folded into the row's final normalisation ("GPT OSS" model notes,
// sections 3 and 4.1).  The causal mask is aligned to the end of the visible
// keys, so a chunk over a cached prefix sees the whole prefix.
//
// Work decomposition: one workgroup (4 waves) owns BM = 128 consecutive query
// rows of one query head of one sequence; wave w owns rows 32w .. 32w+31.  The
// 1-D grid is ordered so that every workgroup of one (sequence, KV head) runs
// on the same XCD (its L2 then serves the K/V tiles to all of them) and the
// query tiles with the most keys start first.  Keys are walked in tiles of
// BN = 64 (four 16-token HND pages), double-buffered in LDS: while a tile is
// multiplied, the next one is loaded into registers (whole rows per lane quad)
// and then written to the other buffer, one barrier per tile.
//
// Per tile and wave, on 32x32x16 bf16 matrix instructions:
//   S^T[32 keys x 32 rows] = K[32 x d] (LDS, row-major) * Q^T[d x 32] (regs)
//   O^T[32 dims x 32 rows] += V^T[32 dims x 16 keys] * P^T[16 keys x 32 rows]
// Lane l holds row l%32 of S^T's columns, so the S^T accumulators are already
// the P^T operand and each row's softmax state stays in its two lanes.  V^T
// comes from the row-major V tile with LDS transpose reads (ds_read_b64_tr_b16:
// within 16 lanes, lane i gets element i%4 of the 8 bytes addressed by lane
// 4j + i/4, j = 0..3, i.e. column i of 4 consecutive rows).  K and V rows are
// stored with XOR-swizzled chunks so that these reads are free of bank
// conflicts.
#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2_t lds_read_tr(const uint16_t *p)
{
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t *)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

// Row sum of packed bf16 pairs (the same rounded weights the PV product uses).
__device__ __forceinline__ float add_pair(uint32_t pair, float acc)
{
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), one, acc, false);
}

__device__ __forceinline__ int load_scalar(const int32_t *p, long long idx)
{
    return ((const __attribute__((address_space(4))) int32_t *)p)[idx];
}

struct PrefillArgs {
    const uint16_t *__restrict__ q;
    const uint16_t *__restrict__ k_cache;
    const uint16_t *__restrict__ v_cache;
    const int32_t *__restrict__ block_table;
    const int32_t *__restrict__ seq_lens;
    const int32_t *__restrict__ cu_seqlens_q;
    const float *__restrict__ sinks;
    uint16_t *__restrict__ out;
    int num_seqs, num_q_heads, num_kv_heads, group, max_pages, num_q_tiles;
    int xcd_groups;  // (sequence, KV head) groups laid out XCD by XCD
    float scale_log2;
};

// LDS tile layouts (bf16 elements).  K: 16-byte chunk c of key row r stored at
// chunk c ^ ksw(r); V: 8-byte chunk c stored at c ^ vsw(r).
template <int D>
struct Tile {
    static __device__ __forceinline__ int k_at(int key, int chunk16)
    {
        const int sw = D == 64 ? ((key >> 1) & 7) : (key & 15);
        return key * D + ((chunk16 ^ sw) << 3);
    }
    static __device__ __forceinline__ int v_at(int key, int chunk8)
    {
        const int sw = D == 64 ? (((key >> 1) & 3) << 2) : ((key & 7) << 2);
        return key * D + ((chunk8 ^ sw) << 2);
    }
    uint16_t k[kBN * D];
    uint16_t v[kBN * D];
};

// Registers of one K/V tile in flight: each thread holds 16-byte chunks
// c = tid + 256 i of the row-major tile (key c / (D/8), chunk c % (D/8)).
template <int D>
struct TileRegs {
    static constexpr int kPer = kBN * D / 8 / kThreads;
    u32x4_t k[kPer];
    u32x4_t v[kPer];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D> &tr, const PrefillArgs &a,
                                          const int32_t *__restrict__ bt, int kv0, int L, int g)
{
    constexpr size_t slab = 16 * D;
    // the tile's four pages (scalar loads); pages past the sequence are not read
    int pages[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        pages[j] = kv0 + 16 * j < L ? load_scalar(bt, (kv0 >> 4) + j) : 0;
#pragma unroll
    for (int i = 0; i < TileRegs<D>::kPer; ++i) {
        const int c = threadIdx.x + kThreads * i;
        const int key = c / (D / 8), chunk = c % (D / 8);
        const int pj = key >> 4;
        const int page = pj == 0 ? pages[0] : pj == 1 ? pages[1] : pj == 2 ? pages[2] : pages[3];
        const size_t off = ((size_t)page * a.num_kv_heads + g) * slab + (key & 15) * D + chunk * 8;
        if (kv0 + key < L) {
            tr.k[i] = *(const u32x4_t *)(a.k_cache + off);
            tr.v[i] = *(const u32x4_t *)(a.v_cache + off);
        } else {  // rows past the sequence are zero (they may hold NaN in memory)
            tr.k[i] = u32x4_t{0, 0, 0, 0};
            tr.v[i] = u32x4_t{0, 0, 0, 0};
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(Tile<D> &t, const TileRegs<D> &tr)
{
#pragma unroll
    for (int i = 0; i < TileRegs<D>::kPer; ++i) {
        const int c = threadIdx.x + kThreads * i;
        const int key = c / (D / 8), chunk = c % (D / 8);
        *(u32x4_t *)&t.k[Tile<D>::k_at(key, chunk)] = tr.k[i];
        // the two 8-byte halves stay adjacent: the V swizzle keeps bit 0
        *(u32x4_t *)&t.v[Tile<D>::v_at(key, 2 * chunk)] = tr.v[i];
    }
}

template <int D>
struct RowState {
    u32x4_t qop[D / 16];     // Q^T operand: row l%32, dims 16kk + 8(l/32) .. +7
    f32x16_t acc[D / 32];    // O^T: dims 32db + 8(r/4) + 4(l/32) + r%4 of row l%32
    float m;                 // reference maximum, base-2 units
    float lsum;              // this lane's half of the row sum
    int pos;                 // position of the row (its last visible key)
};

template <int D, bool kMasked>
__device__ __forceinline__ void compute_tile(RowState<D> &rs, const Tile<D> &t, int kv0, int L,
                                             float scale_log2, int lane)
{
    const int r32 = lane & 31, half = lane >> 5;
    // S^T for the two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const u32x4_t kop = *(const u32x4_t *)&t.k[Tile<D>::k_at(kb * 32 + r32, 2 * kk + half)];
            s[kb] = mfma32x32x16(kop, rs.qop[kk], s[kb]);
        }
    }
    if (kMasked) {
        const int lim = min(rs.pos, L - 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kv0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3) > lim)
                    s[kb][r] = kNegInf;
    }
    // row maximum over the tile (raw scores; the scale is positive)
    float bm = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            bm = fmaxf(bm, s[kb][r]);
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64)) * scale_log2;
    const float m_new = (bm > rs.m + kRescaleSlack) ? bm : rs.m;
    if (__any(m_new != rs.m)) {
        const float alpha = exp2_fast(rs.m - m_new);
        rs.lsum *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            rs.acc[db] *= alpha;
        rs.m = m_new;
    }
    // a row whose keys are all masked so far keeps m = -inf and weights 0
    const float neg_m = rs.m == kNegInf ? 0.f : -rs.m;
    u32x4_t pop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int kb = ks >> 1, r0 = 8 * (ks & 1);
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p0 = exp2_fast(fmaf(s[kb][r0 + 2 * j], scale_log2, neg_m));
            const float p1 = exp2_fast(fmaf(s[kb][r0 + 2 * j + 1], scale_log2, neg_m));
            w[j] = pack_bf16(p0, p1);
            rs.lsum = add_pair(w[j], rs.lsum);
        }
        pop[ks] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
    // O^T += V^T * P^T; V^T operand by transpose reads of the row-major tile
    const int g16 = lane >> 4, i16 = lane & 15;
    const int src_key = 4 * half + (i16 >> 2);        // row of this lane's 8-byte read
    const int src_dim = 16 * (g16 & 1) + 4 * (i16 & 3);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int key = 16 * ks + src_key;
            const int dim = 32 * db + src_dim;
            const u32x2_t lo = lds_read_tr(&t.v[Tile<D>::v_at(key, dim >> 2)]);
            const u32x2_t hi = lds_read_tr(&t.v[Tile<D>::v_at(key + 8, dim >> 2)]);
            const u32x4_t aop = {lo[0], lo[1], hi[0], hi[1]};
            rs.acc[db] = mfma32x32x16(aop, pop[ks], rs.acc[db]);
        }
}

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_bf16(PrefillArgs a)
{
    // workgroup -> (sequence, KV head, query head in group, query tile): all
    // workgroups of one (sequence, KV head) land on one XCD (workgroups are
    // dispatched to XCDs round-robin), heaviest query tiles first
    const int per_group = a.group * a.num_q_tiles;
    const int id = blockIdx.x;
    int grp, r;
    const int main_ids = a.xcd_groups * per_group;
    if (id < main_ids) {
        const int xcd = id & 7, k = id >> 3;
        grp = xcd + 8 * (k / per_group);
        r = k % per_group;
    } else {
        grp = a.xcd_groups + (id - main_ids) / per_group;
        r = (id - main_ids) % per_group;
    }
    const int b = grp / a.num_kv_heads, g = grp % a.num_kv_heads;
    const int qt = a.num_q_tiles - 1 - r / a.group;
    const int h = g * a.group + r % a.group;

    const int q0 = a.cu_seqlens_q[b];
    const int q_len = a.cu_seqlens_q[b + 1] - q0;
    const int row0 = qt * kBM;
    if (row0 >= q_len)
        return;  // uniform over the workgroup
    const int L = a.seq_lens[b];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r32 = lane & 31, half = lane >> 5;
    const int shift = L - q_len;  // position of query row i is shift + i

    RowState<D> rs;
    const int row = row0 + 32 * wave + r32;
    rs.pos = shift + row;
    rs.m = kNegInf;
    rs.lsum = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
        rs.acc[db] = f32x16_t{};
    if (row < q_len) {
        const uint16_t *qrow = a.q + ((size_t)(q0 + row) * a.num_q_heads + h) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            rs.qop[kk] = *(const u32x4_t *)(qrow + 16 * kk + 8 * half);
    } else {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            rs.qop[kk] = u32x4_t{0, 0, 0, 0};
    }

    // keys needed by the workgroup and by this wave
    const int last_row = min(row0 + kBM, q_len) - 1;
    const int kv_end = min(shift + last_row + 1, L);
    const int wave_first = row0 + 32 * wave;
    const int wave_last = min(wave_first + 31, q_len - 1);
    const int wave_kv_end = wave_first < q_len ? min(shift + wave_last + 1, L) : 0;
    const int wave_pos_first = shift + wave_first;

    __shared__ Tile<D> tiles[2];
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    const int ntiles = (kv_end + kBN - 1) / kBN;
    TileRegs<D> regs;
    load_tile<D>(regs, a, bt, 0, L, g);
    store_tile<D>(tiles[0], regs);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int kv0 = it * kBN;
        if (it + 1 < ntiles)
            load_tile<D>(regs, a, bt, kv0 + kBN, L, g);
        if (kv0 < wave_kv_end) {
            const Tile<D> &t = tiles[it & 1];
            if (kv0 + kBN - 1 > wave_pos_first || kv0 + kBN > L)
                compute_tile<D, true>(rs, t, kv0, L, a.scale_log2, lane);
            else
                compute_tile<D, false>(rs, t, kv0, L, a.scale_log2, lane);
        }
        if (it + 1 < ntiles)
            store_tile<D>(tiles[(it + 1) & 1], regs);
        __syncthreads();
    }

    const float sink2 = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
    const float lsum = rs.lsum + __shfl_xor(rs.lsum, 32, 64);
    const float M = fmaxf(rs.m, sink2);
    float scale = 0.f;
    if (M != kNegInf) {
        const float f = rs.m == kNegInf ? 0.f : exp2_fast(rs.m - M);
        const float den = lsum * f + (sink2 == kNegInf ? 0.f : exp2_fast(sink2 - M));
        scale = den > 0.f ? f / den : 0.f;
    }
    if (row < q_len) {
        uint16_t *orow = a.out + ((size_t)(q0 + row) * a.num_q_heads + h) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const u32x2_t w = {pack_bf16(rs.acc[db][4 * r4] * scale,
                                             rs.acc[db][4 * r4 + 1] * scale),
                                   pack_bf16(rs.acc[db][4 * r4 + 2] * scale,
                                             rs.acc[db][4 * r4 + 3] * scale)};
                *(u32x2_t *)(orow + 32 * db + 8 * r4 + 4 * half) = w;
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
    a.num_seqs = p.num_seqs;
    a.num_q_heads = p.num_q_heads;
    a.num_kv_heads = p.num_kv_heads;
    a.group = p.num_q_heads / p.num_kv_heads;
    a.max_pages = p.max_pages_per_seq;
    a.num_q_tiles = (p.max_q_len + kBM - 1) / kBM;
    const int groups = p.num_seqs * p.num_kv_heads;
    a.xcd_groups = groups / 8 * 8;
    a.scale_log2 = p.scale * kLog2e;
    const long long wgs = (long long)groups * a.group * a.num_q_tiles;
    if (wgs > 0x7fffffffLL)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_bf16<D>, dim3((unsigned)wgs), dim3(kThreads), 0, p.stream, a);
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
