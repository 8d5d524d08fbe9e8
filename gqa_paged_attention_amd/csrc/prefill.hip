// Causal prefill for paged GQA attention with per-head sinks (bf16, gfx950).
//
// Each query row runs the online softmax of "GPT-OSS on day 0" (section
// "Sink Attention": running maximum and sum over blocks of keys) and the sink
// is folded into the row's final normalisation ("GPT OSS" model notes,
// sections 3 and 4.1).  The causal mask is aligned to the end of the visible
// keys, so a chunk over a cached prefix sees the whole prefix.
//
// Work decomposition.  Each wave owns NRB row blocks of 32 rows (d = 64:
// NRB = 2; d = 128: NRB = 1).  With a group size divisible by 4 a workgroup
// of 4 waves takes the same rows (64 at d = 64, 32 at d = 128) of four query
// heads of one KV head (every wave sees the same keys and masks, and each K/V
// tile serves four heads); otherwise its 4 waves take consecutive row blocks
// of one query head (BM = 256 rows at d = 64, 128 at d = 128).  The 1-D grid is ordered so
// that every workgroup of one (sequence, KV head) runs on the same XCD (its
// L2 then serves the K/V tiles to all of them) and the query tiles with the
// most keys start first.
//
// Sliding window.  At d = 64 with four heads per workgroup the windowed
// prefill runs on this pipeline, over the tiles from the one holding the
// oldest key the workgroup's rows see, with a band mask and a reference
// maximum taken lazily (a row's first blocks may hold none of its keys).
// Other shapes run prefill_window_bf16, whose waves stream their own blocks.
//
// Keys are consumed in blocks of 32.  Per block, row block and wave, on
// 32x32x16 bf16 matrix instructions:
//   S^T[32 keys x 32 rows] = K[32 x d] (LDS, row-major) * Q^T[d x 32] (regs)
//   O^T[32 dims x 32 rows] += V^T[32 dims x 16 keys] * P^T[16 keys x 32 rows]
// Lane l holds row l%32 of S^T's columns, so the S^T accumulators are already
// the P^T operand and each row's softmax state stays in its two lanes (l and
// l^32, joined by a permlane32 swap).  The K and V^T operands read from LDS
// serve all NRB row blocks of the wave, which is what keeps the LDS read rate
// below the matrix rate at d = 64.  V^T comes from the row-major V tile with
// LDS transpose reads (ds_read_b64_tr_b16: within 16 lanes, lane i gets
// element i%4 of the 8 bytes addressed by lane 4j + i/4, i.e. column i of 4
// consecutive rows).
//
// K/V reach LDS by direct global-to-LDS loads (no registers): tiles of BN
// keys (64 at d = 64, 32 at d = 128; 16 KiB of K+V either way) rotate through
// S LDS stages (4 at d = 64, 5 at d = 128), issued two tiles ahead.  Each
// 1 KiB load instruction covers whole key rows of one 16-token page; lanes
// fetch the 16-byte chunk that belongs in their slot of the XOR-swizzled row,
// so the transposed and column reads above are free of bank conflicts.  Rows
// past the sequence are fetched as copies of its last row (finite), and the
// causal mask hides them.
//
// Softmax reference.  A row's reference maximum m is set exactly from its
// first block and then kept: weights 2^(s - m) may exceed 1, which bf16 and
// the fp32 accumulators absorb as long as they stay far from overflow.  The
// running row sum (needed anyway) detects the rare row that comes too close
// (sum > 2^64, or not finite); the wave then recomputes its rows after the
// loop with the plain online softmax (exact block maxima, rescaling).  The
// final division uses the same m, so the result does not depend on it.
//
// Pipeline.  At d = 128, step b of a wave issues S^T of block b+1 and P*V of
// block b-1 on the matrix cores while the vector ALU computes the weights of
// block b from the S^T of the previous step; no instruction of a step waits
// for another of the same step, so one wave keeps both pipes busy.  At d = 64
// the two row blocks of a wave run half a step apart (skew_step): each
// half-step pairs the weights of one row block with 8 matrix instructions of
// the other, which needs one S^T register set per row block and leaves room
// to read every LDS operand a step before its use.  At the step that first
// reads tile T, the wave waits for tile T, meets the other waves and issues
// tile T+2.
#include "common.h"
#include "kernels.h"
#include "split.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kKB = 32;          // keys per block: one 32x32 S^T tile
constexpr float kLn2 = 0.693147180559945309417f;
// A running row sum (per lane) above this triggers the exact recompute.
constexpr float kWeightSumLimit = 18446744073709551616.0f;  // 2^64

template <int D>
struct Cfg {
    static constexpr int kNRB = D == 64 ? 2 : 1;        // row blocks per wave
    static constexpr int kBM = 32 * kNRB * kWaves;      // rows per workgroup
    static constexpr int kBN = D == 64 ? 64 : 32;       // keys per LDS tile
    static constexpr int kBPT = kBN / kKB;              // blocks per tile
    static constexpr int kRowsPerLoad = 1024 / (2 * D); // key rows per 1 KiB load
    static constexpr int kTileElems = kBN * D;          // bf16 elements of K (or V) per tile
    // 1 KiB direct loads of one tensor per tile, and per wave
    static constexpr int kChunks = kTileElems * 2 / 1024;
    static constexpr int kChunksPerWave = kChunks / kWaves;
    // LDS stages: a step reads K two blocks ahead of the V it reads, and tile
    // T+2 is issued at the step that starts reading tile T, so the stage it
    // overwrites must have been read for the last time before that step.
    static constexpr int kStages = kBPT == 2 ? 4 : 5;
    static constexpr int kLdsBytes = 2 * kStages * kTileElems * 2;
};

// Blocks after which the LDS stage pattern repeats.
template <int D>
constexpr int kLdsCycle = Cfg<D>::kBPT * Cfg<D>::kStages;

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

// v of lane l and of lane l ^ 32 (the two lanes that hold one row).
__device__ __forceinline__ void halves(float v, float &x, float &y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

// Wait until this wave's direct loads of tile T have landed in LDS (those of
// tile T+1, issued after them, may still be in flight: 2 kChunksPerWave
// loads), then meet the other waves.  The loads are not tracked by the
// compiler's own wait insertion, hence the explicit wait.
template <int kLoadsPerTile>
__device__ __forceinline__ void wait_loads_and_sync(bool all_landed)
{
    static_assert(kLoadsPerTile == 2 || kLoadsPerTile == 4, "loads per tile");
    if (all_landed)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (kLoadsPerTile == 4)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    // the LDS wait through the builtin, so that the compiler knows every
    // earlier LDS read has landed and adds no wait for them later
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
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
    int window;      // sliding window W (keys p - W + 1 .. p), 0: none
    // Ragged cache-free mode: K/V rows [tokens][Hkv][d] with per-sequence
    // offsets cu_seqlens_kv (NULL: the paged cache above), row stride
    // kv_stride = Hkv d elements.
    const int32_t *__restrict__ cu_seqlens_kv;
    int kv_stride;
    int causal;        // 1: bottom-right causal; 0: every row sees all keys
    float *__restrict__ lse;  // [total_q][Hq] natural-log row LSE (sink included), or NULL
    float scale_log2;
    // The one-launch mixed batch only: workgroups [0, split_wgs) run the
    // split pass of its decode rows with these arguments (split_wgs_x of them
    // per KV-head group); the prefill's own workgroups follow.
    split::SplitArgs split;
    int split_wgs_x, split_wgs;
};

// LDS tile layouts (bf16 elements).  K: 16-byte chunk c of key row r stored at
// slot c ^ ksw(r); V: 8-byte chunk c stored at c ^ vsw(r), where vsw is even
// so 16-byte chunks stay whole.  Both keep every access of the kernel free of
// bank conflicts whether the LDS serves 8 lanes x 16 B (128 B) or 16 lanes x
// 16 B (256 B) per cycle: the K column reads (32 consecutive rows, one chunk),
// the 1 KiB tile writes and the V transpose reads (4 consecutive rows x 32 or
// 64 bytes).
template <int D>
struct Swz {
    static __device__ __forceinline__ int ksw(int key)
    {
        return D == 64 ? (((key >> 1) & 7) ^ ((key & 1) << 2)) : (key & 15);
    }
    static __device__ __forceinline__ int vsw(int key)
    {
        // d = 128: (bits 3,2) and (bits 4,3) of the four patterns both differ
        return D == 64 ? ((key & 3) << 2) : ((0x18140c00 >> (8 * (key & 3))) & 0xff);
    }
    static __device__ __forceinline__ int k_at(int key, int chunk16)
    {
        return key * D + ((chunk16 ^ ksw(key)) << 3);
    }
    static __device__ __forceinline__ int v_at(int key, int chunk8)
    {
        return key * D + ((chunk8 ^ vsw(key)) << 2);
    }
};

// LDS: the K stages, then the V stages (dynamic shared memory, kLdsBytes).
template <int D>
struct Smem {
    uint16_t *base;
    __device__ __forceinline__ uint16_t *k(int stage) const
    {
        return base + stage * Cfg<D>::kTileElems;
    }
    __device__ __forceinline__ uint16_t *v(int stage) const
    {
        return base + (Cfg<D>::kStages + stage) * Cfg<D>::kTileElems;
    }
};

// Per-lane parts of this wave's direct loads (constant over tiles).  With NW
// waves sharing the loads, the wave loads 1 KiB chunks j = wave + NW i
// (i < kChunks / NW) of each K and V tile; chunk j holds
// key rows R*j .. R*j+R-1 (R = 1024 / (2 d)), all inside one 16-token page,
// and lane l fetches the 16-byte chunk that belongs in slot l % (d/8) of row
// R*j + l / (d/8) of the swizzled tile.
template <int D, int NW = kWaves>
struct LoadLanes {
    static constexpr int kPer = Cfg<D>::kChunks / NW;  // chunks per wave and tensor
    int key[kPer];  // key of this lane's row within the tile, per chunk
    int kc[kPer];   // K chunk (elements) within the row
    int vc[kPer];   // V chunk (elements) within the row
    // byte offsets of this lane's K and V chunks in a tile that lies wholly
    // inside the sequence: from the chunk's page slab (paged), or from the
    // tile's first key row (contiguous rows kv_stride apart)
    uint32_t ko[kPer], vo[kPer];
};

template <int D, bool kContig, int NW = kWaves>
__device__ __forceinline__ LoadLanes<D, NW> load_lanes(int wave, int lane, int kv_stride)
{
    using C = Cfg<D>;
    constexpr int kChunks = D / 8;  // 16-byte chunks per key row
    LoadLanes<D, NW> ll;
#pragma unroll
    for (int i = 0; i < LoadLanes<D, NW>::kPer; ++i) {
        const int j = wave + NW * i;
        const int key = C::kRowsPerLoad * j + lane / kChunks;
        const int slot = lane % kChunks;
        ll.key[i] = key;
        ll.kc[i] = 8 * (slot ^ Swz<D>::ksw(key));
        ll.vc[i] = 8 * (slot ^ (Swz<D>::vsw(key) >> 1));
        const uint32_t row = kContig ? (uint32_t)key * (uint32_t)kv_stride : (key & 15) * D;
        ll.ko[i] = 2 * (row + ll.kc[i]);
        ll.vo[i] = 2 * (row + ll.vc[i]);
    }
    return ll;
}

// One direct global-to-LDS load: lane l's 16 bytes at gbase + voff land at
// LDS byte address lds + 16 l.  Issued as inline assembly so that the
// compiler does not tie its own LDS reads to these loads (it would wait for
// every load in flight, the prefetches included); the kernel waits for them
// explicitly (wait_loads_and_sync).  M0 holds the LDS address.  The
// compiler does not look inside the assembly for hazards, so the assembly
// opens with five wait states itself: a vector instruction that wrote the
// base's scalar registers (v_readlane, as when they come back from a spill)
// needs five before a vector-memory instruction reads them, and the write
// of M0 needs one before the load that reads it.
__device__ __forceinline__ void dma16(const uint16_t *gbase, uint32_t voff, const uint16_t *lds)
{
    const uint32_t lds_addr =
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t *)lds;
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(gbase), "{m0}"(lds_addr)
                 : "memory");
}

// Page ids of this wave's load chunks of tile t (chunk j = wave + NW i starts
// at key t*BN + R*j).  Page indices past the sequence's last page are
// clamped to it.  Read one tile before the loads that use them, so that the
// scalar-load latency stays off the tile start.
struct ChunkPages {
    int p[2];
};

// first_page: under a sliding window, the page of the oldest key the
// workgroup sees; chunks on pages below it (wholly outside every window)
// take that page instead, whose table entry is valid (their keys are masked
// either way; load_tile keeps their rows inside the sequence, so the data
// stays finite).
template <int D, int NW = kWaves>
__device__ __forceinline__ ChunkPages chunk_pages(const int32_t *__restrict__ bt, int t,
                                                  int last_page, int wave, int first_page = 0)
{
    using C = Cfg<D>;
    ChunkPages cp;
    cp.p[1] = 0;
#pragma unroll
    for (int i = 0; i < LoadLanes<D, NW>::kPer; ++i)
        cp.p[i] = load_scalar(
            bt, min(max((t * C::kBN + C::kRowsPerLoad * (wave + NW * i)) >> 4, first_page),
                    last_page));
    return cp;
}

// Issue this wave's direct loads of tile t (keys t*BN ..) into stage t % S.
// Rows past the sequence repeat its last row (finite; the causal mask hides
// them); their page index is clamped to the last page, which holds that row.
// A tile wholly inside the sequence takes the lanes' precomputed offsets.
// first_page: the lower page clamp of chunk_pages.  A chunk it moved up
// reads that page's row of the same slot, or the sequence's last row where
// that slot lies past the end (the first page can be the last, partly
// filled one; rows past the end of a page are not the sequence's data).  In
// a tile wholly inside the sequence every row of the first page is inside it.
// kContig: K/V rows are contiguous [tokens][Hkv][d] and kv_off is the element
// offset of the sequence's key 0 for this KV head (the 16-byte chunks of one
// load then come from R rows kv_stride apart).  Paged: kv_off is the head's
// offset inside a page (g * 16 * d).
template <int D, bool kContig, int NW = kWaves>
__device__ __forceinline__ void load_tile(const Smem<D> &sm, const PrefillArgs &a, const ChunkPages &cp,
                                          int t, int L, size_t kv_off, int wave,
                                          const LoadLanes<D, NW> &ll, int first_page = 0)
{
    using C = Cfg<D>;
    constexpr int kPer = LoadLanes<D, NW>::kPer;
    const int kv0 = t * C::kBN;
    const int stage = t % C::kStages;
    if (kv0 + C::kBN <= L) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int j = wave + NW * i;
            const size_t base = kContig ? kv_off + (size_t)kv0 * a.kv_stride
                                        : (size_t)cp.p[i] * a.num_kv_heads * 16 * D + kv_off;
            dma16(a.k_cache + base, ll.ko[i], sm.k(stage) + 512 * j);
            dma16(a.v_cache + base, ll.vo[i], sm.v(stage) + 512 * j);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = wave + NW * i;
        if constexpr (kContig) {
            const int tok = min(kv0 + ll.key[i], L - 1);
            const uint32_t row = (uint32_t)tok * (uint32_t)a.kv_stride;
            dma16(a.k_cache + kv_off, 2 * (row + ll.kc[i]), sm.k(stage) + 512 * j);
            dma16(a.v_cache + kv_off, 2 * (row + ll.vc[i]), sm.v(stage) + 512 * j);
        } else {
            const size_t slab = (size_t)cp.p[i] * a.num_kv_heads * 16 * D + kv_off;
            // the token this lane's row stands for on the page it reads
            const int tok = 16 * max((kv0 + ll.key[i]) >> 4, first_page) + (ll.key[i] & 15);
            const int row = min(tok, L - 1) & 15;
            dma16(a.k_cache + slab, 2 * (row * D + ll.kc[i]), sm.k(stage) + 512 * j);
            dma16(a.v_cache + slab, 2 * (row * D + ll.vc[i]), sm.v(stage) + 512 * j);
        }
    }
}

template <int D>
struct WaveState {
    static constexpr int kNRB = Cfg<D>::kNRB;
    u32x4_t qop[kNRB][D / 16];   // Q^T operand: row l%32, dims 16kk + 8(l/32) .. +7
    f32x16_t acc[kNRB][D / 32];  // O^T: dims 32db + 8(r/4) + 4(l/32) + r%4 of row l%32
    u32x4_t pop[kNRB][2];        // P^T of the block whose P*V is next
    float m[kNRB];               // reference maximum, base-2 units
    float lsum[kNRB];            // this lane's half of the row sum
};

// K operands of keys key0 .. key0+31 of an LDS K tile.
template <int D>
__device__ __forceinline__ void read_k(u32x4_t (&kop)[D / 16], const uint16_t *kt, int key0,
                                       int lane)
{
    const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        kop[kk] = *(const u32x4_t *)&kt[Swz<D>::k_at(key0 + r32, 2 * kk + half)];
}

// V^T operands of keys key0 .. key0+31 of an LDS V tile: vop[db][ks] covers
// dims 32db .. 32db+31 and keys key0 + 16ks + {4h..4h+3, 8+4h..8+4h+3}.
template <int D>
__device__ __forceinline__ void read_v(u32x4_t (&vop)[D / 32][2], const uint16_t *vt, int key0,
                                       int lane)
{
    const int half = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
    const int src_key = 4 * half + (i16 >> 2);        // row of this lane's 8-byte read
    const int src_dim = 16 * (g16 & 1) + 4 * (i16 & 3);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int key = key0 + 16 * ks + src_key;
            const int dim = 32 * db + src_dim;
            const u32x2_t lo = lds_read_tr(&vt[Swz<D>::v_at(key, dim >> 2)]);
            const u32x2_t hi = lds_read_tr(&vt[Swz<D>::v_at(key + 8, dim >> 2)]);
            vop[db][ks] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
}

// Per-lane LDS element offsets of read_k's and read_v's reads within a
// 32-key block (read_k: one per 16-dim slice; read_v: one per 32-dim block,
// the 16-key halves and the +8 rows being constant offsets from it, as the V
// swizzle depends on key % 4 only).  With a block address the compiler knows,
// every read is one of these plus an immediate.
template <int D>
struct LdsLanes {
    int k[D / 16];
    int v[D / 32];
};

template <int D>
__device__ __forceinline__ LdsLanes<D> lds_lanes(int lane)
{
    const int r32 = lane & 31, half = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
    const int src_key = 4 * half + (i16 >> 2);
    const int src_dim = 16 * (g16 & 1) + 4 * (i16 & 3);
    LdsLanes<D> l;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        l.k[kk] = Swz<D>::k_at(r32, 2 * kk + half);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
        l.v[db] = Swz<D>::v_at(src_key, (32 * db + src_dim) >> 2);
    return l;
}

// read_k and read_v (key0 = 0) through precomputed lane offsets.
template <int D>
__device__ __forceinline__ void read_k_at(u32x4_t (&kop)[D / 16], const uint16_t *kt,
                                          const LdsLanes<D> &l)
{
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        kop[kk] = *(const u32x4_t *)(kt + l.k[kk]);
}

template <int D>
__device__ __forceinline__ void read_v_at(u32x4_t (&vop)[D / 32][2], const uint16_t *vt,
                                          const LdsLanes<D> &l)
{
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x2_t lo = lds_read_tr(vt + l.v[db] + 16 * ks * D);
            const u32x2_t hi = lds_read_tr(vt + l.v[db] + (16 * ks + 8) * D);
            vop[db][ks] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
}

template <int D>
__device__ __forceinline__ f32x16_t qk_mfma(const u32x4_t (&qop)[D / 16],
                                            const u32x4_t (&kop)[D / 16])
{
    f32x16_t s = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        s = mfma32x32x16(kop[kk], qop[kk], s);
    return s;
}

template <int D>
__device__ __forceinline__ void pv_mfma(f32x16_t (&acc)[D / 32], const u32x4_t (&vop)[D / 32][2],
                                        const u32x4_t (&pop)[2])
{
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            acc[db] = mfma32x32x16(vop[db][ks], pop[ks], acc[db]);
}

// Keys of the block with offset > thr (the row's position minus the block
// start, minus 4h for h = lane / 32) are invisible.
__device__ __forceinline__ void apply_mask(f32x16_t &s, int thr)
{
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s[r] = 8 * (r >> 2) + (r & 3) > thr ? kNegInf : s[r];
}

// Sliding window: keys with offset > thr or <= thr - W are invisible (the
// window holds the W positions up to the row's own).
__device__ __forceinline__ void apply_band(f32x16_t &s, int thr, int window)
{
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int e = 8 * (r >> 2) + (r & 3);
        s[r] = (e > thr || e <= thr - window) ? kNegInf : s[r];
    }
}

// Exact block maximum of the row, base-2 units.
__device__ __forceinline__ float block_max(const f32x16_t &s, float scale_log2)
{
    float bm = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r)
        bm = fmaxf(bm, s[r]);
    float x, y;
    halves(bm, x, y);
    return fmaxf(x, y) * scale_log2;  // raw scores: the scale is positive
}

// Weights 2^(s*scale_log2 - m) of one S^T block as the P^T operands of its
// two 16-key halves (pop[ks]: keys 16ks + {4h..4h+3, 8+4h..8+4h+3} of this
// lane's row, the k order of the V^T operand); returns sum plus their sum
// (this lane).
__device__ __forceinline__ float block_weights(const f32x16_t &s, float m, u32x4_t (&pop)[2],
                                               float scale_log2, float sum)
{
    const float neg_m = -m;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        uint32_t pw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p0 = exp2_fast(fmaf(s[8 * ks + 2 * j], scale_log2, neg_m));
            const float p1 = exp2_fast(fmaf(s[8 * ks + 2 * j + 1], scale_log2, neg_m));
            pw[j] = pack_bf16(p0, p1);
            sum = add_pair(pw[j], sum);
        }
        pop[ks] = u32x4_t{pw[0], pw[1], pw[2], pw[3]};
    }
    return sum;
}

// LDS position of block j: stage (j / BPT) % S, key offset 32 (j % BPT).
template <int D>
__device__ __forceinline__ const uint16_t *k_block(const Smem<D> &sm, int j)
{
    using C = Cfg<D>;
    return sm.k((j / C::kBPT) % C::kStages) + kKB * (j % C::kBPT) * D;
}

template <int D>
__device__ __forceinline__ const uint16_t *v_block(const Smem<D> &sm, int j)
{
    using C = Cfg<D>;
    return sm.v((j / C::kBPT) % C::kStages) + kKB * (j % C::kBPT) * D;
}

// S^T of one block for every row block, kk-interleaved so that the row
// blocks' dependent chains overlap in the matrix pipe.
template <int D>
__device__ __forceinline__ void qk_all(f32x16_t (&s)[Cfg<D>::kNRB], const WaveState<D> &w,
                                       const u32x4_t (&kop)[D / 16])
{
#pragma unroll
    for (int rb = 0; rb < Cfg<D>::kNRB; ++rb)
        s[rb] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int rb = 0; rb < Cfg<D>::kNRB; ++rb)
            s[rb] = mfma32x32x16(kop[kk], w.qop[rb][kk], s[rb]);
}

// Step b of one wave.  kQK: S^T of block b+1 into s_next (the caller swaps
// the two S^T register sets between steps).  kPV: P*V of block
// b-1 with the weights in w.pop.  Always: the weights of block b from s_cur,
// relative to the reference maxima (set from the block itself when kFirst,
// masked when kMasked).  A wave with a row sum too close to overflow (or
// not finite) after the loop is recomputed exactly (exact_rows), so the
// loop itself has no rescale branch.  kPhase >= 0: b is
// known to be kPhase modulo the LDS cycle (BPT * S blocks), so the operands'
// LDS addresses are compile-time constants.
template <int D, bool kQK, bool kPV, bool kMasked, bool kFirst, int kPhase = -1>
__device__ __forceinline__ void step(WaveState<D> &w, const Smem<D> &sm, int b,
                                     f32x16_t (&s_cur)[Cfg<D>::kNRB],
                                     f32x16_t (&s_next)[Cfg<D>::kNRB], int thr0, float scale_log2,
                                     int lane, int rb_step,
                                     const LdsLanes<D> *lanes = nullptr)
{
    constexpr int NRB = Cfg<D>::kNRB;
    u32x4_t kop[D / 16], vop[D / 32][2];
    if constexpr (kPhase >= 0) {
        if (kQK)
            read_k_at<D>(kop, k_block<D>(sm, kPhase + 1), *lanes);
        if (kPV)
            read_v_at<D>(vop, v_block<D>(sm, kPhase - 1 + kLdsCycle<D>), *lanes);
    } else {
        if (kQK)
            read_k<D>(kop, k_block<D>(sm, b + 1), 0, lane);
        if (kPV)
            read_v<D>(vop, v_block<D>(sm, b - 1), 0, lane);
    }
    if (kQK)
        qk_all<D>(s_next, w, kop);
    if (kPV) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
            pv_mfma<D>(w.acc[rb], vop, w.pop[rb]);
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        if (kMasked)
            apply_mask(s_cur[rb], thr0 + rb_step * rb);
        // the first block sets the reference exactly; key 0 is visible to
        // every row, so it is finite from then on
        if (kFirst)
            w.m[rb] = block_max(s_cur[rb], scale_log2);
        w.lsum[rb] = block_weights(s_cur[rb], w.m[rb], w.pop[rb], scale_log2, w.lsum[rb]);
        // Keep the weights in this step: without a use here, the compiler
        // moves their computation to the next use, past the branch of the
        // next tile start, where it no longer overlaps this step's matrix
        // instructions.
        asm volatile("" ::"v"(w.pop[rb][0]), "v"(w.pop[rb][1]), "v"(w.lsum[rb]));
    }
    if (kQK && kPV && D == 64) {
        // vector work first while the LDS reads land, then one matrix
        // instruction per eight vector ones (at d = 128, with twice the
        // matrix work per weight, the compiler's own order does better)
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
        for (int i = 0; i < 8 * NRB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
    }
}

// Step nb: P*V of the wave's last block.
template <int D>
__device__ __forceinline__ void last_step(WaveState<D> &w, const Smem<D> &sm, int nb, int lane)
{
    u32x4_t vop[D / 32][2];
    read_v<D>(vop, v_block<D>(sm, nb - 1), 0, lane);
#pragma unroll
    for (int rb = 0; rb < Cfg<D>::kNRB; ++rb)
        pv_mfma<D>(w.acc[rb], vop, w.pop[rb]);
}

// ---- skewed row blocks -----------------------------------------------------
// The two row blocks of a wave run half a step apart, so that every half-step
// pairs the vector work of one row block with matrix work of the other:
//   half A of step b: weights of block b for row block 1, while S^T of block
//                     b+1 for row block 0 and P*V of block b for row block 0
//                     go to the matrix cores;
//   half B of step b: weights of block b+1 for row block 0, while S^T of
//                     block b+1 and P*V of block b for row block 1 do.
// Each row block then needs one S^T register set (its weights are taken
// before its next S^T is written), and each half-step has 8 matrix
// instructions to overlap with about 50 vector ones.  The K operands of
// block b+2 are read into the second K register set at the start of step b
// (a whole step ahead), the V operands of block b+1 at its end.  Every row's
// arithmetic is that of the plain order, so the results are the same bits.

template <int D>
__device__ __forceinline__ void qk_rb(f32x16_t &s, const u32x4_t (&qop)[D / 16],
                                      const u32x4_t (&kop)[D / 16])
{
    s = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        s = mfma32x32x16(kop[kk], qop[kk], s);
}

// Weights of one row block (mask, reference maximum on the first block).
template <bool kMasked, bool kFirst>
__device__ __forceinline__ void weights_rb(float &m, float &lsum, u32x4_t (&pop)[2], f32x16_t &s,
                                           int thr, float scale_log2)
{
    if (kMasked)
        apply_mask(s, thr);
    if (kFirst)
        m = block_max(s, scale_log2);
    lsum = block_weights(s, m, pop, scale_log2, lsum);
    asm volatile("" ::"v"(pop[0]), "v"(pop[1]), "v"(lsum));
}

// Step b.  kNext: block b+1 exists (S^T of it, weights of it for row block
// 0); kMasked: the weights need the causal mask; kFirst: b = 0 (row block 1
// takes its reference maximum from it).  kcur: K of block b+1; knext:
// receives K of block b+2 (kReadK); vop: V of block b, then of block b+1
// (kReadV).  thr: the row's position minus 4 (lane / 32), for block 0.
template <int D, bool kNext, bool kMasked, bool kFirst, bool kReadK, bool kReadV,
          int kPhase = -1>
__device__ __forceinline__ void skew_step(WaveState<D> &w, const Smem<D> &sm, int b,
                                          f32x16_t (&s)[2], const u32x4_t (&kcur)[D / 16],
                                          u32x4_t (&knext)[D / 16], u32x4_t (&vop)[D / 32][2],
                                          int thr, int rbs, float sl2, int lane,
                                          const LdsLanes<D> *lanes = nullptr)
{
    static_assert(Cfg<D>::kNRB == 2, "two row blocks");
    if (kReadK) {
        if constexpr (kPhase >= 0)
            read_k_at<D>(knext, k_block<D>(sm, kPhase + 2), *lanes);
        else
            read_k<D>(knext, k_block<D>(sm, b + 2), 0, lane);
    }
    // half A
    if (kNext)
        qk_rb<D>(s[0], w.qop[0], kcur);
    pv_mfma<D>(w.acc[0], vop, w.pop[0]);
    weights_rb<kMasked, kFirst>(w.m[1], w.lsum[1], w.pop[1], s[1], thr - kKB * b + rbs, sl2);
    if (D == 64) {
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // half B
    if (kNext)
        qk_rb<D>(s[1], w.qop[1], kcur);
    pv_mfma<D>(w.acc[1], vop, w.pop[1]);
    if (kNext)
        weights_rb<kMasked, false>(w.m[0], w.lsum[0], w.pop[0], s[0], thr - kKB * (b + 1), sl2);
    if (kReadV) {
        if constexpr (kPhase >= 0)
            read_v_at<D>(vop, v_block<D>(sm, kPhase + 1), *lanes);
        else
            read_v<D>(vop, v_block<D>(sm, b + 1), 0, lane);
    }
    if (D == 64 && kNext) {
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
    }
}

// Weights of one row block under a sliding window: the band mask (keys
// past the row or before its window) when `masked`; when `lazy`, a row that
// has seen no key yet takes its reference maximum from this block (rows whose
// window starts later still have none: their weights are 0).
__device__ __forceinline__ void win_weights_rb(float &m, float &lsum, u32x4_t (&pop)[2],
                                               f32x16_t &s, int thr, int window, bool masked,
                                               bool lazy, float scale_log2)
{
    if (masked)
        apply_band(s, thr, window);
    if (lazy) {
        const float bm = block_max(s, scale_log2);
        m = m == kNegInf ? bm : m;
    }
    const float m_ref = m == kNegInf ? 0.f : m;
    lsum = block_weights(s, m_ref, pop, scale_log2, lsum);
    asm volatile("" ::"v"(pop[0]), "v"(pop[1]), "v"(lsum));
}

// Whether any of the 32 rows at positions p .. p+31 sees a key of block blk
// under a sliding window (row q sees q - window + 1 .. q).
__device__ __forceinline__ bool win_sees(int blk, int p, int window)
{
    return kKB * blk <= p + 31 && kKB * blk + kKB - 1 >= p - window + 1;
}

// skew_step under a sliding window (runtime mask and first-key flags; the
// few blocks of a window do not repay compile-time variants).  Row block 0's
// rows start at position p0; row block 1's at p0 + 32.
template <int D, bool kEdges>
__device__ __forceinline__ void win_step(WaveState<D> &w, const Smem<D> &sm, int b, bool next,
                                         f32x16_t (&s)[2], const u32x4_t (&kcur)[D / 16],
                                         u32x4_t (&knext)[D / 16], u32x4_t (&vop)[D / 32][2],
                                         int thr, int p0, int window, float sl2, int lane)
{
    // a block needs the band mask unless every row of the row block sees
    // all of its keys; a row block's rows have all seen a key after block
    // (p + 32 - window) / 32 of its last row p
    auto masked = [&](int blk, int p) {
        return !(kKB * blk >= p + 32 - window && kKB * blk + kKB - 1 <= p);
    };
    auto lazy = [&](int blk, int p) { return kKB * blk <= max(p + 32 - window, 0); };
    // kEdges: row block rb (rows p0 + 32 rb ..) skips the blocks none of its
    // rows sees (all weights 0): its S^T, weights and P*V of them.  Steps
    // where both row blocks see both blocks run without these branches.
    const bool cur0 = !kEdges || win_sees(b, p0, window);
    const bool cur1 = !kEdges || win_sees(b, p0 + 32, window);
    const bool next0 = next && (!kEdges || win_sees(b + 1, p0, window));
    const bool next1 = next && (!kEdges || win_sees(b + 1, p0 + 32, window));
    if (next)
        read_k<D>(knext, k_block<D>(sm, b + 2), 0, lane);
    if (next0)
        qk_rb<D>(s[0], w.qop[0], kcur);
    if (cur0)
        pv_mfma<D>(w.acc[0], vop, w.pop[0]);
    if (cur1)
        win_weights_rb(w.m[1], w.lsum[1], w.pop[1], s[1], thr - kKB * b + 32, window,
                       masked(b, p0 + 32), lazy(b, p0 + 32), sl2);
    __builtin_amdgcn_sched_barrier(0);
    if (next1)
        qk_rb<D>(s[1], w.qop[1], kcur);
    if (cur1)
        pv_mfma<D>(w.acc[1], vop, w.pop[1]);
    if (next0)
        win_weights_rb(w.m[0], w.lsum[0], w.pop[0], s[0], thr - kKB * (b + 1), window,
                       masked(b + 1, p0), lazy(b + 1, p0), sl2);
    if (next)
        read_v<D>(vop, v_block<D>(sm, b + 1), 0, lane);
}

// One 32-key block of K and V fetched straight from the paged cache: kPer
// 16-byte chunks of each per lane (key c / (d/8), chunk c % (d/8) for c =
// lane + 64 i).  Keys past the sequence repeat its last key (finite; masked).
template <int D>
struct RawBlock {
    static constexpr int kPer = kKB * (D / 8) / 64;
    u32x4_t k[kPer], v[kPer];
};

// k0 is a multiple of 32, so a block spans two pages, whose ids the wave
// reads once (scalar loads); chunk i lies on the first when i < kPer / 2.
// k_lo: the oldest key any row of the wave sees.  When the block's first page
// lies wholly below it (a sliding window), that page's table entry is not
// read and its chunks take rows of the second page instead, kept inside the
// sequence (that page may be its last, partly filled one): finite values
// for keys every row masks.
template <int D, bool kContig = false>
__device__ __forceinline__ void fetch_block(RawBlock<D> &rb, const PrefillArgs &a,
                                            const int32_t *__restrict__ bt, int L,
                                            size_t kv_off, int k0, int lane, int k_lo = 0)
{
    constexpr int kChunks = D / 8;
    constexpr int kPer = RawBlock<D>::kPer;
    static_assert(kPer % 2 == 0, "half of the chunks on each page");
    size_t slab[2] = {0, 0};  // element offsets of the two pages' head slabs
    // the first page below every window: its chunks stand for keys 16 on
    const bool skip_first = !kContig && k0 + 16 <= k_lo;
    if constexpr (!kContig) {
        const size_t page_elems = (size_t)a.num_kv_heads * 16 * D;
        slab[1] = (size_t)load_scalar(bt, min(k0 + 16, L - 1) >> 4) * page_elems + kv_off;
        slab[0] = skip_first
                      ? slab[1]
                      : (size_t)load_scalar(bt, min(k0, L - 1) >> 4) * page_elems + kv_off;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int c = lane + 64 * i;
        const int key = c / kChunks, chunk = c % kChunks;
        const int tok = min(k0 + key + (skip_first && i < kPer / 2 ? 16 : 0), L - 1);
        size_t off;
        if constexpr (kContig)
            off = kv_off + (size_t)tok * a.kv_stride + 8 * chunk;
        else
            off = slab[i < kPer / 2 ? 0 : 1] + (size_t)(tok & 15) * D + 8 * chunk;
        rb.k[i] = *(const u32x4_t *)(a.k_cache + off);
        rb.v[i] = *(const u32x4_t *)(a.v_cache + off);
    }
}

// Into a wave's own K and V tiles (32 keys each, the layouts of the pipelined
// loop), then wait until the wave's writes are done.
template <int D>
__device__ __forceinline__ void stash_block(const RawBlock<D> &rb, uint16_t *kt, uint16_t *vt,
                                            int lane)
{
    constexpr int kChunks = D / 8;
#pragma unroll
    for (int i = 0; i < RawBlock<D>::kPer; ++i) {
        const int c = lane + 64 * i;
        const int key = c / kChunks, chunk = c % kChunks;
        *(u32x4_t *)&kt[Swz<D>::k_at(key, chunk)] = rb.k[i];
        *(u32x4_t *)&vt[Swz<D>::v_at(key, 2 * chunk)] = rb.v[i];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// Plain online softmax over one block held in the wave's tiles: exact row
// maximum, running state rescaled to it, weights, P*V.  kBand: sliding-window
// mask (both sides) instead of the causal one.  A row that has seen no
// visible key yet keeps m = -inf and adds nothing (its weights are 0).
template <int D, bool kBand>
__device__ __forceinline__ void exact_block(WaveState<D> &w, const uint16_t *kt,
                                            const uint16_t *vt, bool masked, int thr,
                                            int window, float scale_log2, int lane,
                                            int rb_step = 32)
{
    u32x4_t kop[D / 16], vop[D / 32][2];
    read_k<D>(kop, kt, 0, lane);
    read_v<D>(vop, vt, 0, lane);
#pragma unroll
    for (int rb = 0; rb < Cfg<D>::kNRB; ++rb) {
        f32x16_t s = qk_mfma<D>(w.qop[rb], kop);
        if (kBand)
            apply_band(s, thr + rb_step * rb, window);
        else if (masked)
            apply_mask(s, thr + rb_step * rb);
        const float m_new = fmaxf(w.m[rb], block_max(s, scale_log2));
        const float m_ref = m_new == kNegInf ? 0.f : m_new;
        const float alpha = exp2_fast(w.m[rb] - m_ref);  // 0 while m is -inf
        w.lsum[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            w.acc[rb][db] *= alpha;
        w.m[rb] = m_new;
        w.lsum[rb] = block_weights(s, m_ref, w.pop[rb], scale_log2, w.lsum[rb]);
        pv_mfma<D>(w.acc[rb], vop, w.pop[rb]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next block's writes
    __builtin_amdgcn_wave_barrier();
}

// One block of the windowed prefill: the online softmax of exact_block with
// a lazy maximum (raised only when a block's maximum exceeds it by more than
// kRescaleSlack, so weights stay below 2^kRescaleSlack), which spares the
// rescale of the accumulators on almost every block.  The block holds keys
// k0 .. k0+31; the wave's rows sit at positions wpf + 32 rb + (0 .. 31); a
// row block that sees none of the keys skips the block, and one that sees
// all of them skips the band mask.
template <int D>
__device__ __forceinline__ void window_block(WaveState<D> &w, const uint16_t *kt,
                                             const uint16_t *vt, int thr, int window, int k0,
                                             int wpf, float scale_log2, int lane)
{
    u32x4_t kop[D / 16], vop[D / 32][2];
    read_k<D>(kop, kt, 0, lane);
    read_v<D>(vop, vt, 0, lane);
#pragma unroll
    for (int rb = 0; rb < Cfg<D>::kNRB; ++rb) {
        const int p_first = wpf + 32 * rb;
        // no key of the block in any row's window: nothing to do
        if (k0 > p_first + 31 || k0 + kKB - 1 < p_first - window + 1)
            continue;
        f32x16_t s = qk_mfma<D>(w.qop[rb], kop);
        if (!(k0 + kKB - 1 <= p_first && k0 >= p_first + 31 - window + 1))
            apply_band(s, thr + 32 * rb, window);
        const float bm = block_max(s, scale_log2);
        const float m_new = bm > w.m[rb] + kRescaleSlack ? bm : w.m[rb];
        if (__any(m_new != w.m[rb])) {
            // 0 on a row's first visible block (its state is empty)
            const float alpha = m_new == w.m[rb] ? 1.f : exp2_fast(w.m[rb] - m_new);
            w.lsum[rb] *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                w.acc[rb][db] *= alpha;
            w.m[rb] = m_new;
        }
        const float m_ref = w.m[rb] == kNegInf ? 0.f : w.m[rb];
        w.lsum[rb] = block_weights(s, m_ref, w.pop[rb], scale_log2, w.lsum[rb]);
        pv_mfma<D>(w.acc[rb], vop, w.pop[rb]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next block's writes
    __builtin_amdgcn_wave_barrier();
}

// Exact recompute of a wave's rows (rare: some row sum came too close to
// overflow against the reference taken from the first block).  K and V come
// straight from the paged cache into this wave's own part of the LDS (the
// workgroup has met after its pipelined loop, so nothing else reads it).
template <int D, bool kContig>
__device__ void exact_rows(WaveState<D> &w, uint16_t *lds_wave, const PrefillArgs &a,
                           const int32_t *__restrict__ bt, int L, size_t kv_off, int nb,
                           int wpf, int thr, int rb_step, int lane, int window = 0, int j0 = 0)
{
    constexpr int NRB = Cfg<D>::kNRB;
    uint16_t *kt = lds_wave;
    uint16_t *vt = lds_wave + kKB * D;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        w.m[rb] = kNegInf;
        w.lsum[rb] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            w.acc[rb][db] = f32x16_t{};
    }
    const int k_lo = window > 0 ? max(wpf - window + 1, 0) : 0;
    for (int blk = j0; blk < nb; ++blk) {
        const int k0 = kKB * blk;
        RawBlock<D> raw;
        fetch_block<D, kContig>(raw, a, bt, L, kv_off, k0, lane, k_lo);
        stash_block<D>(raw, kt, vt, lane);
        if (window > 0)
            exact_block<D, true>(w, kt, vt, true, thr - k0, window, a.scale_log2, lane, rb_step);
        else
            exact_block<D, false>(w, kt, vt, k0 + kKB - 1 > wpf, thr - k0, 0, a.scale_log2, lane,
                                  rb_step);
    }
}

// Workgroup -> (sequence, KV head, first query head, query tile): all
// workgroups of one (sequence, KV head) land on one XCD (workgroups are
// dispatched to XCDs round-robin), heaviest query tiles first.  A workgroup
// takes HPW consecutive query heads of the KV head.
struct TileCoords {
    int b, g, h, qt;
};

template <int HPW, bool kMixed = false>
__device__ __forceinline__ TileCoords tile_of(const PrefillArgs &a)
{
    const int hgroups = a.group / HPW;
    const int per_group = hgroups * a.num_q_tiles;
    const int id = kMixed ? (int)blockIdx.x - a.split_wgs : (int)blockIdx.x;
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
    TileCoords tc;
    tc.b = grp / a.num_kv_heads;
    tc.g = grp % a.num_kv_heads;
    tc.qt = a.num_q_tiles - 1 - r / hgroups;
    tc.h = tc.g * a.group + HPW * (r % hgroups);
    return tc;
}

// Q^T operands of the wave's rows (rows past the chunk read its last row and
// are never stored); the running state starts empty.
template <int D>
__device__ __forceinline__ void init_rows(WaveState<D> &w, const PrefillArgs &a, int q0, int q_len,
                                          int row_w, int h, int lane)
{
    const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int rb = 0; rb < Cfg<D>::kNRB; ++rb) {
        const int row = row_w + 32 * rb + r32;
        w.m[rb] = kNegInf;
        w.lsum[rb] = 0.f;
        w.pop[rb][0] = w.pop[rb][1] = u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            w.acc[rb][db] = f32x16_t{};
        const uint16_t *qrow = a.q + ((size_t)(q0 + min(row, q_len - 1)) * a.num_q_heads + h) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            w.qop[rb][kk] = row < q_len ? *(const u32x4_t *)(qrow + 16 * kk + 8 * half)
                                        : u32x4_t{0, 0, 0, 0};
    }
}

// The head's sink logit in base-2 units (-inf without sinks).  Read when a
// wave starts, so that its latency overlaps the first loads instead of
// delaying the epilogue.
__device__ __forceinline__ float sink_log2(const PrefillArgs &a, int h)
{
    return a.sinks ? a.sinks[h] * kLog2e : kNegInf;
}

// Epilogue: fold the sink (sink2, from sink_log2) into each row's
// normalisation, then write the wave's rows through its own LDS staging area
// (32 NRB rows of d bf16) so that every global store covers whole 16-byte
// chunks of contiguous output rows.  The staging rows are XOR-swizzled by
// 16-byte chunk (both the 8-byte writes and the 16-byte reads are then free
// of bank conflicts).
template <int D>
__device__ __forceinline__ void store_rows(const WaveState<D> &w, uint16_t *stage,
                                           const PrefillArgs &a, int q0, int q_len, int row_w,
                                           int h, int lane, float sink2)
{
    constexpr int NRB = Cfg<D>::kNRB;
    constexpr int kC16 = D / 8;  // 16-byte chunks per row
    const int r32 = lane & 31, half = lane >> 5;
    auto st_at = [&](int r, int c16) { return r * D + 8 * (c16 ^ (r & (kC16 - 1))); };
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        float lx, ly;
        halves(w.lsum[rb], lx, ly);
        const float lsum = lx + ly;
        const float M = fmaxf(w.m[rb], sink2);
        float scale = 0.f, lse = kNegInf;
        if (M != kNegInf) {
            const float f = w.m[rb] == kNegInf ? 0.f : exp2_fast(w.m[rb] - M);
            const float den = lsum * f + (sink2 == kNegInf ? 0.f : exp2_fast(sink2 - M));
            scale = den > 0.f ? f / den : 0.f;
            // natural log of the row's softmax denominator, sink included
            if (den > 0.f)
                lse = (M + __builtin_amdgcn_logf(den)) * kLn2;
        }
        // lane l holds dims 32 db + 8 r4 + 4 (l/32) .. +3 of row 32 rb + l%32
        const int r = 32 * rb + r32;
        if (a.lse && half == 0 && row_w + r < q_len)
            a.lse[(size_t)(q0 + row_w + r) * a.num_q_heads + h] = lse;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x16_t &o = w.acc[rb][db];
                const u32x2_t v = {pack_bf16(o[4 * r4] * scale, o[4 * r4 + 1] * scale),
                                   pack_bf16(o[4 * r4 + 2] * scale, o[4 * r4 + 3] * scale)};
                *(u32x2_t *)&stage[st_at(r, 4 * db + r4) + 4 * half] = v;
            }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
    __builtin_amdgcn_wave_barrier();
    // 64 lanes copy 64 / kC16 rows per pass, kC16 lanes per row
    constexpr int kRowsPerPass = 64 / kC16;
#pragma unroll
    for (int r0 = 0; r0 < 32 * NRB; r0 += kRowsPerPass) {
        const int r = r0 + lane / kC16, c16 = lane % kC16;
        const int row = row_w + r;
        const u32x4_t v = *(const u32x4_t *)&stage[st_at(r, c16)];
        if (row < q_len)
            *(u32x4_t *)(a.out + ((size_t)(q0 + row) * a.num_q_heads + h) * D + 8 * c16) = v;
    }
}

// kContig: ragged cache-free attention over contiguous K/V rows (with or
// without the causal mask); otherwise the paged cache.  kWaitAll: the tile
// waits take every load of the wave (vmcnt(0)) instead of leaving the next
// tile's in flight (a debug setting; same results).  HPW: query heads per
// workgroup.  With HPW = 1 the 4 waves take consecutive row blocks of one
// head (BM rows); with HPW = 4 they take the same 32 NRB rows of 4 heads of
// one KV head, so every wave sees the same keys, masks and block count (no
// wave waits at the tile barriers for the others' extra diagonal blocks) and
// the causal range of a workgroup's tiles is 4 times finer.
// kMixed: the mixed batch in one launch.  Its first a.split_wgs workgroups
// run the split pass of the batch's single-token decode rows instead (as
// decode_split_bf16 runs it: workgroup id % split_wgs_x of KV-head group
// id / split_wgs_x), so that they are dispatched before the prefill's
// workgroups fill the chip and the memory-bound pass runs beside the
// compute-bound one; the others run the prefill of its chunks.
template <int D, bool kContig, bool kWaitAll, int HPW, bool kWin = false, bool kMixed = false>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16(PrefillArgs a)
{
    static_assert(!kWin || (D == 64 && HPW == 4 && !kContig), "windowed layout");
    static_assert(!kMixed || (!kContig && !kWin), "mixed batch: paged, causal, no window");
    if constexpr (kMixed) {
        if ((int)blockIdx.x < a.split_wgs) {
            // waves past the workgroup's KV heads have no work (the split
            // pass has no barrier)
            if ((int)(threadIdx.x >> 6) < a.split.heads_per_wg)
                split::split_body<D, 1>(a.split, split::FlatIdx{(unsigned)a.split_wgs_x});
            return;
        }
    }
    using C = Cfg<D>;
    constexpr int NRB = C::kNRB;
    constexpr int kWavesPerHead = kWaves / HPW;
    constexpr int kRowsPerWg = 32 * NRB * kWavesPerHead;
    const TileCoords tc = tile_of<HPW, kMixed>(a);
    const int b = tc.b, g = tc.g, qt = tc.qt;

    const int q0 = a.cu_seqlens_q[b];
    const int q_len = a.cu_seqlens_q[b + 1] - q0;
    const int row0 = qt * kRowsPerWg;
    if (row0 >= q_len)
        return;  // uniform over the workgroup
    const int kv_first = kContig ? a.cu_seqlens_kv[b] : 0;
    const int L = kContig ? a.cu_seqlens_kv[b + 1] - kv_first : a.seq_lens[b];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = tc.h + wave / kWavesPerHead;
    const float sink2 = sink_log2(a, h);
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, half = lane >> 5;
    // Position of query row i: shift + i (causal, aligned to the end of the
    // keys); without the causal mask every row is treated as the last
    // position, L - 1, so that it sees all keys.
    const bool causal = !kContig || a.causal;
    const int shift = L - q_len;
    const int row_step = causal ? 1 : 0;
    const int rbs = 32 * row_step;  // position step between row blocks

    // this wave's rows: row_w + 32 rb + r32
    const int row_w = row0 + 32 * NRB * (wave % kWavesPerHead);

    // keys needed by the workgroup (tiles) and by this wave (blocks)
    const int last_row = min(row0 + kRowsPerWg, q_len) - 1;
    const int kv_end = causal ? min(shift + last_row + 1, L) : L;
    const int ntiles = (kv_end + C::kBN - 1) / C::kBN;
    const int wave_last = min(row_w + 32 * NRB - 1, q_len - 1);
    const int nb = row_w < q_len
                       ? ((causal ? min(shift + wave_last + 1, L) : L) + kKB - 1) / kKB
                       : 0;
    // position of the wave's first row
    const int wpf = causal ? shift + row_w : L - 1;

    extern __shared__ __align__(16) uint16_t lds[];
    const Smem<D> sm{lds};
    const int32_t *bt = kContig ? nullptr : a.block_table + (size_t)b * a.max_pages;
    const int last_page = (L - 1) >> 4;
    // the KV head's data: element offset of its key 0 (contiguous rows), or
    // its offset inside a page
    const size_t kv_off = kContig ? (size_t)kv_first * a.kv_stride + (size_t)g * D
                                  : (size_t)g * 16 * D;
    // Sliding window: the workgroup's rows (the same for its 4 waves) see
    // keys from k_lo on; its tiles start at the tile of k_lo, its blocks at
    // that tile's first block j0, and pages below k_lo's are never read.
    const int window = kWin ? a.window : 0;
    const int k_lo = kWin ? max(wpf - window + 1, 0) : 0;
    const int t_lo = k_lo / C::kBN;
    const int j0 = C::kBPT * t_lo;

    // tiles t_lo and t_lo+1 in flight before the loop; tile T+2 is issued
    // when the wave starts reading tile T
    const LoadLanes<D> ll = load_lanes<D, kContig>(wave, lane, a.kv_stride);
    auto pages = [&](int t) {
        if constexpr (kContig)
            return ChunkPages{{0, 0}};
        else
            return chunk_pages<D>(bt, t, last_page, wave, k_lo >> 4);
    };
    // Q first (its rows need only the chunk offsets), then the first tiles
    // (whose page ids take one more round trip), so that the Q loads are in
    // flight during that round trip; one wait covers both (the compiler then
    // knows the Q registers are ready and adds no waits inside the loops)
    WaveState<D> w;
    init_rows<D>(w, a, q0, q_len, row_w, h, lane);
#pragma unroll
    for (int t = 0; t < 2; ++t)
        if (t_lo + t < ntiles)
            load_tile<D, kContig>(sm, a, pages(t_lo + t), t_lo + t, L, kv_off, wave, ll,
                                      k_lo >> 4);
    ChunkPages next_pages = pages(t_lo + 2);

    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

    // blocks from bm on hold keys past the wave's first row: causal mask
    const int bm = (wpf + 1) / kKB;
    const int thr = wpf + row_step * r32 - 4 * half;  // minus the block start
    if constexpr (NRB == 2) {
    // Step j reads K of block j+2 (tile (j+2)/BPT) and V of block j+1.  When
    // block j+2 starts tile T, the wave first waits for tile T, meets the
    // other waves and issues tile T+2 (steps -2 and -1 do this for tiles 0
    // and 1).  Waves with fewer blocks keep doing so after their last step.
    auto tile_start = [&](int step) {
        if ((step + 2) % C::kBPT == 0) {
            const int t = (step + 2) / C::kBPT;
            if (t < ntiles) {
                // the page ids of tile t+3 are read before the wait, which
                // covers them: no scalar load is in flight afterwards, so the
                // compiler can wait for LDS reads by count
                const ChunkPages later = pages(t + 3);
                wait_loads_and_sync<2 * C::kChunksPerWave>(kWaitAll || t + 1 >= ntiles);
                if (t + 2 < ntiles)
                    load_tile<D, kContig>(sm, a, next_pages, t + 2, L, kv_off, wave, ll,
                                          k_lo >> 4);
                next_pages = later;
            }
        }
    };
    const float sl2 = a.scale_log2;
    const LdsLanes<D> lane_ofs = lds_lanes<D>(lane);
    f32x16_t s[NRB];
    u32x4_t ka[D / 16], kb[D / 16], vop[D / 32][2];
    if constexpr (kWin) {
        // blocks j0 .. nb-1 (a window's few blocks), masks and first-key
        // references decided per block
        tile_start(j0 - 2);
        tile_start(j0 - 1);
        read_k<D>(ka, k_block<D>(sm, j0), 0, lane);
        if (win_sees(j0, wpf, window))
            qk_rb<D>(s[0], w.qop[0], ka);
        if (win_sees(j0, wpf + 32, window))
            qk_rb<D>(s[1], w.qop[1], ka);
        read_k<D>(ka, k_block<D>(sm, j0 + 1), 0, lane);
        read_v<D>(vop, v_block<D>(sm, j0), 0, lane);
        if (win_sees(j0, wpf, window))
            win_weights_rb(w.m[0], w.lsum[0], w.pop[0], s[0], thr - kKB * j0, window, true, true,
                           sl2);
        // Steps in pairs (K of the next block alternates between ka and
        // kb): first those with blocks row block 1 does not see, then those
        // whose three blocks j .. j+2 both row blocks see (row block 1's
        // oldest block lo1 on, up to row block 0's newest, hi0), then the
        // rest.
        const int lo1 = max(wpf + 32 - window + 1, 0) / kKB, hi0 = (wpf + 31) / kKB;
        int j = j0;
        auto pair = [&](auto edges) {
            constexpr bool kEdges = decltype(edges)::value;
            tile_start(j);
            win_step<D, kEdges>(w, sm, j, j + 1 < nb, s, ka, kb, vop, thr, wpf, window, sl2,
                                lane);
            if (j + 1 < nb) {
                tile_start(j + 1);
                win_step<D, kEdges>(w, sm, j + 1, j + 2 < nb, s, kb, ka, vop, thr, wpf, window,
                                    sl2, lane);
            }
            j += 2;
        };
        while (j < nb && j < lo1)
            pair(std::true_type{});
        while (j + 1 < nb && j + 2 <= hi0)
            pair(std::false_type{});
        while (j < nb)
            pair(std::true_type{});
        for (int j = nb; j + 2 <= C::kBPT * ntiles; ++j)
            tile_start(j);
    } else {
    tile_start(-2);
    tile_start(-1);
    if (nb > 0) {
        // S^T of block 0 for both row blocks, weights of row block 0; the
        // operands of step 0 (K of block 1, V of block 0)
        read_k<D>(ka, k_block<D>(sm, 0), 0, lane);
        qk_rb<D>(s[0], w.qop[0], ka);
        qk_rb<D>(s[1], w.qop[1], ka);
        read_k<D>(ka, k_block<D>(sm, 1), 0, lane);
        read_v<D>(vop, v_block<D>(sm, 0), 0, lane);
        if (bm == 0)
            weights_rb<true, true>(w.m[0], w.lsum[0], w.pop[0], s[0], thr, sl2);
        else
            weights_rb<false, true>(w.m[0], w.lsum[0], w.pop[0], s[0], thr, sl2);
    }
    // step 0 (row block 1 takes its reference maximum from block 0)
    tile_start(0);
    if (nb > 1) {
        if (bm <= 1)
            skew_step<D, true, true, true, true, true>(w, sm, 0, s, ka, kb, vop, thr, rbs, sl2,
                                                       lane);
        else
            skew_step<D, true, false, true, true, true>(w, sm, 0, s, ka, kb, vop, thr, rbs, sl2,
                                                        lane);
    } else if (nb == 1) {
        skew_step<D, false, true, true, false, false>(w, sm, 0, s, ka, kb, vop, thr, rbs, sl2,
                                                      lane);
    }
    // Steps 1 .. nb-2 in pairs (odd steps take K from kb and read into ka,
    // even ones the other way round); steps whose weights reach the diagonal
    // run the masked variant.  Then the last step.
    int j = 1;
    const int steady_end = min(bm - 1, nb - 1);  // steps before it need no mask
    if constexpr (kLdsCycle<D> == 8) {
        for (; j + 7 < steady_end; j += 8) {
            const int jj = (j & ~7) | 1;  // == j, with its low bits visible
            LdsLanes<D> lr = lane_ofs;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                asm volatile("" : "+v"(lr.k[kk]));
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                asm volatile("" : "+v"(lr.v[db]));
            tile_start(jj);
            skew_step<D, true, false, false, true, true, 1>(w, sm, jj, s, kb, ka, vop, thr, rbs,
                                                            sl2, lane, &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 1);
            skew_step<D, true, false, false, true, true, 2>(w, sm, jj + 1, s, ka, kb, vop, thr,
                                                            rbs, sl2, lane, &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 2);
            skew_step<D, true, false, false, true, true, 3>(w, sm, jj + 2, s, kb, ka, vop, thr,
                                                            rbs, sl2, lane, &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 3);
            skew_step<D, true, false, false, true, true, 4>(w, sm, jj + 3, s, ka, kb, vop, thr,
                                                            rbs, sl2, lane, &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 4);
            skew_step<D, true, false, false, true, true, 5>(w, sm, jj + 4, s, kb, ka, vop, thr,
                                                            rbs, sl2, lane, &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 5);
            skew_step<D, true, false, false, true, true, 6>(w, sm, jj + 5, s, ka, kb, vop, thr,
                                                            rbs, sl2, lane, &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 6);
            skew_step<D, true, false, false, true, true, 7>(w, sm, jj + 6, s, kb, ka, vop, thr,
                                                            rbs, sl2, lane, &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 7);
            skew_step<D, true, false, false, true, true, 0>(w, sm, jj + 7, s, ka, kb, vop, thr,
                                                            rbs, sl2, lane, &lr);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    for (; j + 1 < steady_end; j += 2) {
        tile_start(j);
        skew_step<D, true, false, false, true, true>(w, sm, j, s, kb, ka, vop, thr, rbs, sl2, lane);
        tile_start(j + 1);
        skew_step<D, true, false, false, true, true>(w, sm, j + 1, s, ka, kb, vop, thr, rbs, sl2,
                                                     lane);
    }
    for (; j + 1 < nb - 1; j += 2) {
        tile_start(j);
        skew_step<D, true, true, false, true, true>(w, sm, j, s, kb, ka, vop, thr, rbs, sl2, lane);
        tile_start(j + 1);
        skew_step<D, true, true, false, true, true>(w, sm, j + 1, s, ka, kb, vop, thr, rbs, sl2,
                                                    lane);
    }
    // an odd count of full steps leaves one (K of block j+1 in kb)
    if (j < nb - 1) {
        tile_start(j);
        skew_step<D, true, true, false, true, true>(w, sm, j, s, kb, ka, vop, thr, rbs, sl2, lane);
        ++j;
    }
    // step nb-1: weights of block nb-1 for row block 1, P*V of block nb-1
    // (no S^T or K operands left to take, so the K register set is moot)
    if (nb > 1) {
        tile_start(nb - 1);
        skew_step<D, false, true, false, false, false>(w, sm, nb - 1, s, ka, kb, vop, thr, rbs,
                                                       sl2, lane);
    }
    for (j = max(nb, 1); j + 2 <= C::kBPT * ntiles; ++j)
        tile_start(j);
    }
    } else {
    // Step j reads K of block j+1 (tile (j+1)/BPT) and V of block j-1.  When
    // block j+1 starts tile T, the wave first waits for tile T, meets the
    // other waves and issues tile T+2 (step -1 does this for tile 0).  Waves
    // with fewer blocks keep doing so after their last step.  The first
    // step, the unmasked steps, the masked steps near the diagonal and the
    // last two steps run in separate loops, so each loop body is one
    // straight path.
    auto tile_start = [&](int step) {
        if ((step + 1) % C::kBPT == 0) {
            const int t = (step + 1) / C::kBPT;
            if (t < ntiles) {
                wait_loads_and_sync<2 * C::kChunksPerWave>(kWaitAll || t + 1 >= ntiles);
                if (t + 2 < ntiles) {
                    load_tile<D, kContig>(sm, a, next_pages, t + 2, L, kv_off, wave, ll);
                    next_pages = pages(t + 3);
                }
            }
        }
    };
    const float sl2 = a.scale_log2;
    const LdsLanes<D> lane_ofs = lds_lanes<D>(lane);
    // S^T of the block whose weights are next, and of the one after: two
    // register sets that trade roles every step (the steady loop is unrolled
    // twice so that no copy is needed)
    f32x16_t sa[NRB], sb[NRB];
    tile_start(-1);
    if (nb > 0) {
        u32x4_t kop[D / 16];
        read_k<D>(kop, k_block<D>(sm, 0), 0, lane);
        qk_all<D>(sa, w, kop);
    }
    // step 0
    tile_start(0);
    if (nb > 1) {
        if (bm == 0)
            step<D, true, false, true, true>(w, sm, 0, sa, sb, thr, sl2, lane, rbs);
        else
            step<D, true, false, false, true>(w, sm, 0, sa, sb, thr, sl2, lane, rbs);
    } else if (nb == 1) {
        if (bm == 0)
            step<D, false, false, true, true>(w, sm, 0, sa, sb, thr, sl2, lane, rbs);
        else
            step<D, false, false, false, true>(w, sm, 0, sa, sb, thr, sl2, lane, rbs);
    }
    // Steps 1 .. nb-2: all three stages, in pairs (sb then sa holds the
    // current S^T), so that no register copy is needed; step 0 left S^T of
    // block 1 in sb and every pair leaves the next one there.  An odd count
    // ends with one single step that moves its next S^T into sb.  The pairs
    // that reach the diagonal run the masked variant (a block with no
    // invisible key is unchanged by it).
    int j = 1;
    const int steady_end = min(bm, nb - 1);
    if constexpr (kLdsCycle<D> == 8) {
        // The steady pairs in runs of four.  The pairs start at block 1, so
        // every run starts at a block that is 1 modulo the LDS cycle: its LDS
        // addresses are compile-time constants (no address arithmetic per
        // step).
        for (; j + 7 < steady_end; j += 8) {
            const int jj = (j & ~7) | 1;  // == j, with its low bits visible
            // the lane offsets hidden from the compiler for this run, so that
            // it folds each read's constant block address into the read
            // instead of keeping eight sets of sums live across the run
            LdsLanes<D> lr = lane_ofs;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                asm volatile("" : "+v"(lr.k[kk]));
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                asm volatile("" : "+v"(lr.v[db]));
            tile_start(jj);
            step<D, true, true, false, false, 1>(w, sm, jj, sb, sa, 0, sl2, lane, rbs,
                                                &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 1);
            step<D, true, true, false, false, 2>(w, sm, jj + 1, sa, sb, 0, sl2, lane, rbs,
                                                &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 2);
            step<D, true, true, false, false, 3>(w, sm, jj + 2, sb, sa, 0, sl2, lane, rbs,
                                                &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 3);
            step<D, true, true, false, false, 4>(w, sm, jj + 3, sa, sb, 0, sl2, lane, rbs,
                                                &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 4);
            step<D, true, true, false, false, 5>(w, sm, jj + 4, sb, sa, 0, sl2, lane, rbs,
                                                &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 5);
            step<D, true, true, false, false, 6>(w, sm, jj + 5, sa, sb, 0, sl2, lane, rbs,
                                                &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 6);
            step<D, true, true, false, false, 7>(w, sm, jj + 6, sb, sa, 0, sl2, lane, rbs,
                                                &lr);
            __builtin_amdgcn_sched_barrier(0);
            tile_start(jj + 7);
            step<D, true, true, false, false, 0>(w, sm, jj + 7, sa, sb, 0, sl2, lane, rbs,
                                                &lr);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (kLdsCycle<D> == 5) {
        // One block per tile and five stages (d = 128): runs of ten steps
        // (two LDS cycles, an even count for the register-set swap) from
        // block 1, so every run starts at a block that is 1 modulo the cycle.
        for (; j + 9 < steady_end; j += 10) {
            LdsLanes<D> lr = lane_ofs;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                asm volatile("" : "+v"(lr.k[kk]));
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                asm volatile("" : "+v"(lr.v[db]));
            // two(P): the steps of blocks j+P-1 and j+P, which are P and
            // P+1 modulo the cycle
            auto two = [&](auto p0) {
                constexpr int kP = decltype(p0)::value;
                tile_start(j + kP - 1);
                step<D, true, true, false, false, kP % 5>(w, sm, j + kP - 1, sb, sa, 0, sl2, lane,
                                                          rbs, &lr);
                __builtin_amdgcn_sched_barrier(0);
                tile_start(j + kP);
                step<D, true, true, false, false, (kP + 1) % 5>(w, sm, j + kP, sa, sb, 0, sl2,
                                                                lane, rbs, &lr);
                __builtin_amdgcn_sched_barrier(0);
            };
            two(std::integral_constant<int, 1>{});
            two(std::integral_constant<int, 3>{});
            two(std::integral_constant<int, 5>{});
            two(std::integral_constant<int, 7>{});
            two(std::integral_constant<int, 9>{});
        }
    }
    for (; j + 1 < steady_end; j += 2) {
        tile_start(j);
        step<D, true, true, false, false>(w, sm, j, sb, sa, 0, sl2, lane, rbs);
        tile_start(j + 1);
        step<D, true, true, false, false>(w, sm, j + 1, sa, sb, 0, sl2, lane, rbs);
    }
    for (; j + 1 < nb - 1; j += 2) {
        tile_start(j);
        step<D, true, true, true, false>(w, sm, j, sb, sa, thr - kKB * j, sl2, lane, rbs);
        tile_start(j + 1);
        step<D, true, true, true, false>(w, sm, j + 1, sa, sb, thr - kKB * (j + 1), sl2, lane, rbs);
    }
    // an odd count of full steps leaves one, which moves its next S^T into sb
    // (the masked variant leaves a block with no invisible key unchanged)
    if (j < nb - 1) {
        tile_start(j);
        step<D, true, true, true, false>(w, sm, j, sb, sa, thr - kKB * j, sl2, lane, rbs);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
            sb[rb] = sa[rb];
        ++j;
    }
    // step nb-1: weights of the last block (S^T in sb), P*V of the one before
    if (nb > 1) {
        tile_start(nb - 1);
        if (nb - 1 >= bm)
            step<D, false, true, true, false>(w, sm, nb - 1, sb, sb, thr - kKB * (nb - 1), sl2,
                                              lane, rbs);
        else
            step<D, false, true, false, false>(w, sm, nb - 1, sb, sb, 0, sl2, lane, rbs);
    }
    // step nb: P*V of the last block
    if (nb > 0) {
        tile_start(nb);
        last_step<D>(w, sm, nb, lane);
    }
    for (j = max(nb + 1, 1); j <= C::kBPT * ntiles; ++j)
        tile_start(j);
    }
    __syncthreads();  // every wave is past its last read of the stages
    // A row sum only grows (its terms are >= 0; inf and NaN stay), so one
    // test after the loop finds every row whose sum came too close to
    // overflow (or is not finite) at any step.
    bool bad = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
        bad = bad || !(w.lsum[rb] <= kWeightSumLimit);
    if (__any(bad))
        exact_rows<D, kContig>(w, lds + wave * (C::kLdsBytes / 2 / kWaves), a, bt, L, kv_off, nb,
                               wpf, thr, rbs, lane, window, j0);

    // Epilogue through this wave's part of the (now free) LDS.
    store_rows<D>(w, lds + wave * (C::kLdsBytes / 2 / kWaves), a, q0, q_len, row_w, h, lane,
                  sink2);
}

// Sliding-window prefill ("GPT OSS" model notes, section 4.1: even layers
// attend within a local window of W positions; section 11: the window comes
// with each call).  A row at position p sees keys p - W + 1 .. p, so a wave
// needs only the blocks from its first row's oldest key to its last row:
// few for the windows the notes name (W = 128: at most 7 per wave at d = 64).
// Each wave streams its own blocks from the paged cache into its own LDS
// tiles, the next block in registers while the current one is computed, and
// runs the online softmax on each with a lazy maximum (window_block: a row's
// first blocks may hold none of its keys, so no reference is fixed in
// advance).  The four waves of a workgroup never wait for one another.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_window_bf16(PrefillArgs a)
{
    using C = Cfg<D>;
    constexpr int NRB = C::kNRB;
    const TileCoords tc = tile_of<1>(a);
    const int q0 = a.cu_seqlens_q[tc.b];
    const int q_len = a.cu_seqlens_q[tc.b + 1] - q0;
    const int row0 = tc.qt * C::kBM;
    if (row0 >= q_len)
        return;  // uniform over the workgroup
    const int L = a.seq_lens[tc.b];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float sink2 = sink_log2(a, tc.h);
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, half = lane >> 5;
    const int shift = L - q_len;  // position of query row i is shift + i
    const int row_w = row0 + 32 * NRB * wave;
    const int wpf = shift + row_w;  // position of the wave's first row
    const int wave_last = min(row_w + 32 * NRB - 1, q_len - 1);
    const int nb = row_w < q_len ? (min(shift + wave_last + 1, L) + kKB - 1) / kKB : 0;
    const int b_lo = max(wpf - a.window + 1, 0) / kKB;  // the block of the oldest key

    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t *kt = lds + wave * (2 * kKB * D);
    uint16_t *vt = kt + kKB * D;
    const int32_t *bt = a.block_table + (size_t)tc.b * a.max_pages;
    const size_t head_off = (size_t)tc.g * 16 * D;

    WaveState<D> w;
    init_rows<D>(w, a, q0, q_len, row_w, tc.h, lane);
    const int thr = wpf + r32 - 4 * half;  // minus the block start
    // one register block: stored to LDS, then refilled with the next block,
    // whose loads are in flight while the current one is computed
    // (d = 64; at d = 128 the registers are needed by the block itself, and
    // each block is fetched when its turn comes)
    constexpr bool kAhead = D == 64;
    RawBlock<D> raw;
    const int k_lo = max(wpf - a.window + 1, 0);  // the oldest key a row of the wave sees
    if (kAhead && b_lo < nb)
        fetch_block<D>(raw, a, bt, L, head_off, kKB * b_lo, lane, k_lo);
    for (int blk = b_lo; blk < nb; ++blk) {
        const int k0 = kKB * blk;
        if (!kAhead)
            fetch_block<D>(raw, a, bt, L, head_off, k0, lane, k_lo);
        stash_block<D>(raw, kt, vt, lane);
        if (kAhead && blk + 1 < nb)
            fetch_block<D>(raw, a, bt, L, head_off, k0 + kKB, lane, k_lo);
        window_block<D>(w, kt, vt, thr - k0, a.window, k0, wpf, a.scale_log2, lane);
    }
    // the staging area of the epilogue is the wave's own K tile and more:
    // 32 NRB rows of d bf16 fit in its 2 * 32 * d elements
    store_rows<D>(w, kt, a, q0, q_len, row_w, tc.h, lane, sink2);
}

template <int D>
constexpr int kWindowLdsBytes = kWaves * 2 * kKB * D * 2;

bool prefill_one_head() { return debug_setting(kDebugPrefillOneHead) != 0; }
bool prefill_window_streamed() { return debug_setting(kDebugPrefillWindowStreamed) != 0; }
bool prefill_wait_all() { return debug_setting(kDebugPrefillWaitAll) != 0; }

// more than 64 KiB of LDS (d = 128) has to be allowed once per kernel
template <int D, bool kContig, bool kWaitAll, int HPW, bool kWin = false>
hipError_t launch_causal(const PrefillArgs &a, long long wgs, hipStream_t stream)
{
    constexpr int kLds = Cfg<D>::kLdsBytes;
    static const hipError_t attr = hipFuncSetAttribute(
        (const void *)prefill_bf16<D, kContig, kWaitAll, HPW, kWin>,
        hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((prefill_bf16<D, kContig, kWaitAll, HPW, kWin>), dim3((unsigned)wgs),
                       dim3(kThreads), kLds, stream, a);
    return hipGetLastError();
}

template <int D, int HPW>
long long causal_grid(PrefillArgs &a, const PrefillLaunch &p)
{
    constexpr int kRows = 32 * Cfg<D>::kNRB * (kWaves / HPW);
    a.num_q_tiles = (p.max_q_len + kRows - 1) / kRows;
    return (long long)p.num_seqs * p.num_kv_heads * (a.group / HPW) * a.num_q_tiles;
}

template <int D, int HPW>
hipError_t launch_causal_hpw(PrefillArgs a, const PrefillLaunch &p)
{
    const long long wgs = causal_grid<D, HPW>(a, p);
    if (wgs > 0x7fffffffLL)
        return hipErrorInvalidValue;
    const bool contig = p.cu_seqlens_kv != nullptr, wait_all = prefill_wait_all();
    if (contig)
        return wait_all ? launch_causal<D, true, true, HPW>(a, wgs, p.stream)
                        : launch_causal<D, true, false, HPW>(a, wgs, p.stream);
    return wait_all ? launch_causal<D, false, true, HPW>(a, wgs, p.stream)
                    : launch_causal<D, false, false, HPW>(a, wgs, p.stream);
}

// The windowed prefill on the causal kernel's pipeline (d = 64, paged, four
// query heads per workgroup).
hipError_t launch_window64(PrefillArgs a, const PrefillLaunch &p)
{
    const long long wgs = causal_grid<64, 4>(a, p);
    if (wgs > 0x7fffffffLL)
        return hipErrorInvalidValue;
    return prefill_wait_all() ? launch_causal<64, false, true, 4, true>(a, wgs, p.stream)
                              : launch_causal<64, false, false, 4, true>(a, wgs, p.stream);
}

// The prefill kernels' arguments for a launch description.
template <int D>
PrefillArgs prefill_args(const PrefillLaunch &p)
{
    using C = Cfg<D>;
    PrefillArgs a = {};
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
    a.num_q_tiles = (p.max_q_len + C::kBM - 1) / C::kBM;
    const int groups = p.num_seqs * p.num_kv_heads;
    a.xcd_groups = groups / 8 * 8;
    a.window = p.window;
    a.cu_seqlens_kv = p.cu_seqlens_kv;
    a.kv_stride = p.num_kv_heads * D;
    a.causal = p.causal;
    a.lse = p.lse;
    a.scale_log2 = p.scale * kLog2e;
    return a;
}

template <int D>
hipError_t launch_d(const PrefillLaunch &p)
{
    const PrefillArgs a = prefill_args<D>(p);
    const int groups = p.num_seqs * p.num_kv_heads;
    const long long wgs = (long long)groups * a.group * a.num_q_tiles;
    if (wgs > 0x7fffffffLL)
        return hipErrorInvalidValue;
    if (p.window > 0 && p.window < p.max_seq_len) {
        // a window that leaves out some key of some row (otherwise the
        // causal kernel below computes exactly the same rows)
        if constexpr (D == 64) {
            if (a.group % 4 == 0 && !p.cu_seqlens_kv && !prefill_one_head() &&
                !prefill_window_streamed())
                return launch_window64(a, p);
        }
        static const hipError_t wattr = hipFuncSetAttribute(
            (const void *)prefill_window_bf16<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
            kWindowLdsBytes<D>);
        if (wattr != hipSuccess)
            return wattr;
        hipLaunchKernelGGL(prefill_window_bf16<D>, dim3((unsigned)wgs), dim3(kThreads),
                           kWindowLdsBytes<D>, p.stream, a);
        return hipGetLastError();
    }
    // four query heads per workgroup where the group allows it
    if (a.group % 4 == 0 && !prefill_one_head())
        return launch_causal_hpw<D, 4>(a, p);
    return launch_causal_hpw<D, 1>(a, p);
}

// The mixed batch in one launch: the split pass of the decode part, its
// workgroups rounded up to a multiple of 8 (the extra ones find no KV head
// and return) so that the prefill workgroups keep their XCD grouping, then
// the prefill of the chunks.
template <int D, int HPW>
hipError_t launch_mixed_d(const DecodeLaunch &dp, const PrefillLaunch &pp)
{
    PrefillArgs a = prefill_args<D>(pp);
    const long long pwgs = causal_grid<D, HPW>(a, pp);
    const int split_x = dp.num_wgs;
    const int split_y = (dp.num_kv_heads + dp.heads_per_wg - 1) / dp.heads_per_wg;
    const long long swgs = ((long long)split_x * split_y + 7) / 8 * 8;
    if (split_x <= 0 || dp.heads_per_wg > kWaves || dp.q_max != 1 || pwgs + swgs > 0x7fffffffLL)
        return hipErrorInvalidValue;
    a.split = split::split_args(dp);
    a.split_wgs_x = split_x;
    a.split_wgs = (int)swgs;
    constexpr int kLds = Cfg<D>::kLdsBytes;
    static_assert(split::split_lds_bytes<D>(kDecodeMaxHeadsPerWg) <= (size_t)kLds, "split LDS");
    static const hipError_t attr = hipFuncSetAttribute(
        (const void *)prefill_bf16<D, false, false, HPW, false, true>,
        hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((prefill_bf16<D, false, false, HPW, false, true>),
                       dim3((unsigned)(pwgs + swgs)), dim3(kThreads), kLds, pp.stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_mixed_hpw(const DecodeLaunch &dp, const PrefillLaunch &pp)
{
    if ((pp.num_q_heads / pp.num_kv_heads) % 4 == 0 && !prefill_one_head())
        return launch_mixed_d<D, 4>(dp, pp);
    return launch_mixed_d<D, 1>(dp, pp);
}

}  // namespace

hipError_t launch_mixed_bf16(const DecodeLaunch &dp, const PrefillLaunch &pp)
{
    return pp.head_dim == 64 ? launch_mixed_hpw<64>(dp, pp) : launch_mixed_hpw<128>(dp, pp);
}

hipError_t launch_prefill_bf16(const PrefillLaunch &p)
{
    if (p.num_seqs == 0 || p.max_q_len == 0 || p.total_q == 0)
        return hipSuccess;
    return p.head_dim == 64 ? launch_d<64>(p) : launch_d<128>(p);
}

}  // namespace attn
