// C ABI of the library: host-side checks, launch configuration, dispatch.
// Every check runs before anything is enqueued; see include/attn_sinks.h.
#include "attn_sinks.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstddef>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace {

constexpr int kPageSize = 16;
constexpr int kMaxGroup = 16;
constexpr int kVersion = 100;  // 0.1.0

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool supported_head_dim(int d) { return d == 64 || d == 128; }

// Debug overrides of the split-pass launch shape, read once: the number of
// workgroups per head group (ATTN_SINKS_DECODE_WGS) and the KV heads per
// workgroup (ATTN_SINKS_DECODE_HEADS_PER_WG, 1..8).  Invalid values are
// ignored.
int env_int(const char *name, long lo, long hi)
{
    const char *s = std::getenv(name);
    if (!s)
        return 0;
    const long v = std::strtol(s, nullptr, 10);
    return (v >= lo && v <= hi) ? (int)v : 0;
}

int wgs_override()
{
    static int value = 0;
    static std::once_flag once;
    std::call_once(once, [] { value = env_int("ATTN_SINKS_DECODE_WGS", 1, 1 << 20); });
    return value;
}

int heads_override()
{
    static int value = 0;
    static std::once_flag once;
    std::call_once(once, [] {
        value = env_int("ATTN_SINKS_DECODE_HEADS_PER_WG", 1, attn::kDecodeMaxHeadsPerWg);
    });
    return value;
}

// Debug settings: environment defaults read once, then attn_sinks_set_debug.
std::atomic<int> g_debug[attn::kDebugSettings];
std::once_flag g_debug_once;

void debug_init()
{
    std::call_once(g_debug_once, [] {
        const char *k = std::getenv("ATTN_SINKS_PREFILL_ONE_HEAD");
        g_debug[attn::kDebugPrefillOneHead] = (k && std::strcmp(k, "1") == 0) ? 1 : 0;
        const char *w = std::getenv("ATTN_SINKS_PREFILL_WAIT_ALL");
        g_debug[attn::kDebugPrefillWaitAll] = (w && std::strcmp(w, "1") == 0) ? 1 : 0;
        const char *ws = std::getenv("ATTN_SINKS_PREFILL_WINDOW_STREAMED");
        g_debug[attn::kDebugPrefillWindowStreamed] = (ws && std::strcmp(ws, "1") == 0) ? 1 : 0;
    });
}

struct DecodeShape {
    int heads_per_wg;  // waves per workgroup, one KV head each
    int wgs;           // workgroups per head group
};

// Launch shape of the decode split pass.  Every workgroup takes an equal
// share of the 32-token units, so the count only needs to fill the chip once;
// it is capped by an upper bound of the unit count computed from host
// integers, so the launch never depends on device data and the call can be
// captured into a graph.
DecodeShape decode_shape(int num_seqs, int num_kv_heads, int max_seq_len)
{
    DecodeShape s;
    const int cap = heads_override() ? heads_override() : attn::kDecodeMaxHeadsPerWg;
    s.heads_per_wg = num_kv_heads < cap ? num_kv_heads : cap;
    const int groups = (num_kv_heads + s.heads_per_wg - 1) / s.heads_per_wg;
    const long long units_max = (long long)num_seqs * ((max_seq_len + 31) / 32);
    long long w = wgs_override();
    if (!w) {
        // The same number of workgroups on every CU they use, at least 4
        // waves per CU.  Workgroups of 4 waves use three quarters of the CUs:
        // measured on the gpt-oss, mixed and Qwen-shaped decodes, 192 of them
        // beat 256 (one per CU) by 1.3-2.2 %, and counts that put two on some
        // CUs lose 8-20 %, since every workgroup has an equal share of the
        // units.  Smaller workgroups share CUs and fill all of them.
        const int waves_per_cu = s.heads_per_wg > attn::kDecodeMinWavesPerCU
                                     ? s.heads_per_wg
                                     : attn::kDecodeMinWavesPerCU;
        const long long cus = s.heads_per_wg >= attn::kDecodeMinWavesPerCU
                                  ? (long long)attn::kDeviceCUs * 3 / 4
                                  : (long long)attn::kDeviceCUs;
        const long long total = cus * waves_per_cu / s.heads_per_wg;
        w = total / groups;
        if (w < 1)
            w = 1;
    }
    if (units_max < w)
        w = units_max;
    s.wgs = (int)w;
    return s;
}

// Multi-token decode shapes the split pass takes: G x (query tokens per
// sequence) packed rows per KV head within its column blocks (the same bound
// at both head sizes).
bool multi_packed(int group, int max_q_len)
{
    const int rows = group * max_q_len;
    return group > 0 && max_q_len >= 1 &&
           rows <= attn::kMultiRowsMax;
}

int check_common(int dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                 int page_size, int num_pages, int max_pages_per_seq, int max_seq_len)
{
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16)
        return ATTN_ERR_UNSUPPORTED;
    if (!supported_head_dim(head_dim) || page_size != kPageSize)
        return ATTN_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_pages < 0 ||
        max_pages_per_seq < 0 || max_seq_len < 0)
        return ATTN_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0)
        return ATTN_ERR_SHAPE;
    if (num_q_heads / num_kv_heads > kMaxGroup)
        return ATTN_ERR_UNSUPPORTED;
    // launch grids put sequences and heads on the y/z dimensions (<= 65535)
    if (num_seqs > 65535 || num_q_heads > 65535)
        return ATTN_ERR_SHAPE;
    if ((long long)max_seq_len > (long long)max_pages_per_seq * page_size)
        return ATTN_ERR_SHAPE;
    if (max_seq_len > 0 && num_pages == 0)
        return ATTN_ERR_SHAPE;
    // element offsets of the pool must fit the kernels' 64-bit arithmetic and
    // the per-sequence token index must fit an int
    if ((long long)max_pages_per_seq * page_size > INT_MAX)
        return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

// Workspace: ml [slots][q_max][Hq][2] then, 16-byte aligned, acc
// [slots][q_max][Hq][d] (fp32), with slots = num_seqs + workgroups per head
// group and q_max query rows per sequence (1 for decode).
size_t decode_workspace(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                        int max_seq_len, DecodeShape *shape_out, size_t *acc_offset_floats,
                        int q_max = 1)
{
    const DecodeShape shape = decode_shape(num_seqs, num_kv_heads, max_seq_len);
    if (shape_out)
        *shape_out = shape;
    if (shape.wgs == 0) {
        if (acc_offset_floats)
            *acc_offset_floats = 0;
        return 0;
    }
    const size_t rows = ((size_t)num_seqs + (size_t)shape.wgs) * (size_t)q_max;
    const size_t ml = (rows * num_q_heads * 2 + 3) / 4 * 4;
    if (acc_offset_floats)
        *acc_offset_floats = ml;
    return (ml + rows * num_q_heads * (size_t)head_dim) * sizeof(float);
}

// Checks shared by the decode entry points; fills the launch description.
// `reads_kv`: the call reads q and the page pool; `writes_out`: it writes out.
int prepare_decode(int dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                   int page_size, int num_pages, int max_pages_per_seq, int max_seq_len,
                   const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *block_table, const int32_t *seq_lens, const float *sinks,
                   float scale, int window, void *out, void *workspace, size_t workspace_bytes,
                   void *stream, bool reads_kv, bool writes_out, attn::DecodeLaunch *p)
{
    int rc = check_common(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                          num_pages, max_pages_per_seq, max_seq_len);
    if (rc != ATTN_OK)
        return rc;
    if (!std::isfinite(scale) || window < 0)
        return ATTN_ERR_SHAPE;
    if (num_seqs == 0)
        return ATTN_OK;
    if (!seq_lens || (writes_out && !out))
        return ATTN_ERR_NULL;
    if (reads_kv && (!q || (max_seq_len > 0 && (!k_cache || !v_cache || !block_table))))
        return ATTN_ERR_NULL;
    const void *vec[] = {q, k_cache, v_cache, out, workspace};
    for (const void *ptr : vec)
        if (ptr && !aligned16(ptr))
            return ATTN_ERR_ALIGN;
    const void *words[] = {block_table, seq_lens, sinks};
    for (const void *ptr : words)
        if (ptr && !aligned4(ptr))
            return ATTN_ERR_ALIGN;
    DecodeShape shape;
    size_t acc_offset = 0;
    const size_t need = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                         max_seq_len, &shape, &acc_offset);
    // the fp32 path of attn_sinks_decode works on full rows and needs no scratch
    const bool uses_workspace = !(dtype == ATTN_DTYPE_F32 && reads_kv && writes_out);
    if (uses_workspace && need > 0 && (!workspace || workspace_bytes < need))
        return workspace ? ATTN_ERR_WORKSPACE : ATTN_ERR_NULL;
    p->dtype = dtype;
    p->num_seqs = num_seqs;
    p->num_q_heads = num_q_heads;
    p->num_kv_heads = num_kv_heads;
    p->head_dim = head_dim;
    p->max_pages_per_seq = max_pages_per_seq;
    p->num_wgs = shape.wgs;
    p->heads_per_wg = shape.heads_per_wg;
    p->window = window;
    p->cu_seqlens_q = nullptr;
    p->q_max = 1;
    p->q = q;
    p->k_cache = k_cache;
    p->v_cache = v_cache;
    p->block_table = block_table;
    p->seq_lens = seq_lens;
    p->sinks = sinks;
    p->scale = scale;
    p->out = out;
    float *ws = static_cast<float *>(workspace);
    p->part_ml = ws;
    p->part_acc = ws ? ws + acc_offset : nullptr;
    p->stream = reinterpret_cast<hipStream_t>(stream);
    return ATTN_OK;
}

// Checks of a KV append (beyond those of the attention call it may precede).
int check_append(int dtype, int num_seqs, int num_kv_heads, int head_dim, int page_size,
                 int num_pages, int max_pages_per_seq, int max_seq_len, int total_new,
                 const void *k_new, const void *v_new, const int32_t *block_table,
                 const int32_t *seq_lens, const int32_t *cu_seqlens_new, const void *k_cache,
                 const void *v_cache)
{
    int rc = check_common(dtype, num_seqs, num_kv_heads, num_kv_heads, head_dim, page_size,
                          num_pages, max_pages_per_seq, max_seq_len);
    if (rc != ATTN_OK)
        return rc;
    if (total_new < 0 || (!cu_seqlens_new && total_new != num_seqs))
        return ATTN_ERR_SHAPE;
    if (num_seqs == 0 || total_new == 0)
        return ATTN_OK;
    if (max_seq_len == 0)
        return ATTN_ERR_SHAPE;  // new tokens need a place in some page
    if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !seq_lens)
        return ATTN_ERR_NULL;
    const void *vec[] = {k_new, v_new, k_cache, v_cache};
    for (const void *p : vec)
        if (!aligned16(p))
            return ATTN_ERR_ALIGN;
    const void *words[] = {block_table, seq_lens, cu_seqlens_new};
    for (const void *p : words)
        if (p && !aligned4(p))
            return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

int elem_bytes(int dtype) { return dtype == ATTN_DTYPE_F32 ? 4 : 2; }

// bf16 decode of one token per sequence: the direct kernel when every
// sequence's visible keys are few (a short window that cuts some sequence,
// or a length bound within the same limit), else split + merge.
int run_decode_bf16(const attn::DecodeLaunch &p, int max_seq_len)
{
    if ((p.window > 0 && p.window <= attn::kDirectWindowMax && p.window < max_seq_len) ||
        max_seq_len <= attn::kDirectWindowMax)
        return attn::launch_decode_direct_bf16(p) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
    if (attn::launch_decode_split_bf16(p) != hipSuccess)
        return ATTN_ERR_HIP;
    return attn::launch_decode_merge(p) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Fixed scratch of attn_sinks_decode_noalloc, for callers that cannot
// allocate: the split pass's partial results go here instead of into a
// caller workspace.  Every device the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is used.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's copy of `scratch`.
int scratch_address(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return ATTN_ERR_HIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
        return ATTN_ERR_HIP;
    *ptr = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

int attn::debug_setting(int id)
{
    debug_init();
    return (id >= 0 && id < attn::kDebugSettings) ? g_debug[id].load() : 0;
}

extern "C" {

size_t attn_sinks_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int max_seq_len)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
        !supported_head_dim(head_dim) || num_q_heads % num_kv_heads != 0 ||
        num_q_heads / num_kv_heads > kMaxGroup)
        return 0;
    return decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, nullptr,
                            nullptr);
}

int attn_sinks_decode(int dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int page_size, int num_pages, int max_pages_per_seq, int max_seq_len,
                      const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_table, const int32_t *seq_lens, const float *sinks,
                      float scale, void *out, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    return attn_sinks_decode_window(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                    page_size, num_pages, max_pages_per_seq, max_seq_len, q,
                                    k_cache, v_cache, block_table, seq_lens, sinks, scale, 0, out,
                                    workspace, workspace_bytes, stream);
}

int attn_sinks_decode_window(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                             int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                             int max_seq_len, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_table,
                             const int32_t *seq_lens, const float *sinks, float scale, int window,
                             void *out, void *workspace, size_t workspace_bytes, void *stream)
{
    attn::DecodeLaunch p;
    int rc = prepare_decode(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                            num_pages, max_pages_per_seq, max_seq_len, q, k_cache, v_cache,
                            block_table, seq_lens, sinks, scale, window, out, workspace,
                            workspace_bytes, stream, true, true, &p);
    if (rc != ATTN_OK || num_seqs == 0)
        return rc;
    if (dtype == ATTN_DTYPE_F32) {
        hipError_t e = attn::launch_rows_f32(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             max_pages_per_seq, num_seqs, q, k_cache, v_cache,
                                             block_table, seq_lens, nullptr, sinks, scale, window,
                                             out, p.stream);
        return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
    }
    return run_decode_bf16(p, max_seq_len);
}

int attn_sinks_decode_noalloc(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                              int max_seq_len, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_table,
                              const int32_t *seq_lens, const float *sinks, float scale,
                              int window, void *out, void *stream)
{
    // Every check of attn_sinks_decode_window first, against the fixed
    // scratch's size (a stand-in address: nothing is dereferenced here).
    attn::DecodeLaunch p;
    void *const stand_in = reinterpret_cast<void *>((uintptr_t)256);
    int rc = prepare_decode(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                            num_pages, max_pages_per_seq, max_seq_len, q, k_cache, v_cache,
                            block_table, seq_lens, sinks, scale, window, out, stand_in,
                            kScratchBytes, stream, true, true, &p);
    if (rc == ATTN_ERR_WORKSPACE)
        return ATTN_ERR_SCRATCH;
    if (rc != ATTN_OK || num_seqs == 0)
        return rc;
    if (dtype == ATTN_DTYPE_F32) {
        hipError_t e = attn::launch_rows_f32(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             max_pages_per_seq, num_seqs, q, k_cache, v_cache,
                                             block_table, seq_lens, nullptr, sinks, scale, window,
                                             out, p.stream);
        return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
    }
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != ATTN_OK)
        return rc;
    const ptrdiff_t acc_offset = p.part_acc - p.part_ml;
    p.part_ml = static_cast<float *>(ws);
    p.part_acc = p.part_ml + acc_offset;
    return run_decode_bf16(p, max_seq_len);
}

int attn_sinks_decode_partials(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                               int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                               int max_seq_len, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_table,
                               const int32_t *seq_lens, float scale, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    if (dtype != ATTN_DTYPE_BF16)
        return ATTN_ERR_UNSUPPORTED;
    attn::DecodeLaunch p;
    int rc = prepare_decode(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                            num_pages, max_pages_per_seq, max_seq_len, q, k_cache, v_cache,
                            block_table, seq_lens, nullptr, scale, 0, nullptr, workspace,
                            workspace_bytes, stream, true, false, &p);
    if (rc != ATTN_OK || num_seqs == 0)
        return rc;
    return attn::launch_decode_split_bf16(p) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_sinks_decode_merge(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                            int head_dim, int max_seq_len, const int32_t *seq_lens,
                            const float *sinks, const void *workspace, size_t workspace_bytes,
                            void *out, void *stream)
{
    attn::DecodeLaunch p;
    // the merge reads no KV data: give the page-related checks neutral values
    const int pages = (max_seq_len + kPageSize - 1) / kPageSize;
    int rc = prepare_decode(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, kPageSize,
                            pages > 0 ? pages : 1, pages, max_seq_len, nullptr, nullptr, nullptr,
                            nullptr, seq_lens, sinks, 1.0f, 0, out, const_cast<void *>(workspace),
                            workspace_bytes, stream, false, true, &p);
    if (rc != ATTN_OK || num_seqs == 0)
        return rc;
    return attn::launch_decode_merge(p) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_sinks_prefill(int dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int page_size, int num_pages, int max_pages_per_seq, int total_q,
                       int max_q_len, int max_seq_len, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *block_table, const int32_t *seq_lens,
                       const int32_t *cu_seqlens_q, const float *sinks, float scale, void *out,
                       void *stream)
{
    return attn_sinks_prefill_window(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                     page_size, num_pages, max_pages_per_seq, total_q, max_q_len,
                                     max_seq_len, q, k_cache, v_cache, block_table, seq_lens,
                                     cu_seqlens_q, sinks, scale, 0, out, stream);
}

// Checks of a paged causal prefill call; fills the launch description (the
// bf16 kernels') and returns ATTN_OK, or the error code with nothing
// enqueued.  *empty is set when there is nothing to compute.
static int prepare_prefill(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                           int total_q, int max_q_len, int max_seq_len, const void *q,
                           const void *k_cache, const void *v_cache,
                           const int32_t *block_table, const int32_t *seq_lens,
                           const int32_t *cu_seqlens_q, const float *sinks, float scale,
                           int window, void *out, void *stream, attn::PrefillLaunch *pl,
                           bool *empty)
{
    *empty = false;
    int rc = check_common(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                          num_pages, max_pages_per_seq, max_seq_len);
    if (rc != ATTN_OK)
        return rc;
    if (total_q < 0 || max_q_len < 0 || max_q_len > max_seq_len || max_q_len > total_q)
        return ATTN_ERR_SHAPE;
    if (!std::isfinite(scale) || window < 0)
        return ATTN_ERR_SHAPE;
    if (num_seqs == 0 || total_q == 0) {
        *empty = true;
        return ATTN_OK;
    }
    if (!q || !out || !seq_lens || !cu_seqlens_q || !k_cache || !v_cache || !block_table)
        return ATTN_ERR_NULL;
    const void *vec[] = {q, k_cache, v_cache, out};
    for (const void *p : vec)
        if (p && !aligned16(p))
            return ATTN_ERR_ALIGN;
    const void *words[] = {block_table, seq_lens, cu_seqlens_q, sinks};
    for (const void *p : words)
        if (p && !aligned4(p))
            return ATTN_ERR_ALIGN;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    attn::PrefillLaunch &p = *pl;
    p.dtype = dtype;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.head_dim = head_dim;
    p.max_pages_per_seq = max_pages_per_seq;
    p.total_q = total_q;
    p.max_q_len = max_q_len;
    p.max_seq_len = max_seq_len;
    p.window = window;
    p.cu_seqlens_kv = nullptr;
    p.causal = 1;
    p.lse = nullptr;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.cu_seqlens_q = cu_seqlens_q;
    p.sinks = sinks;
    p.scale = scale;
    p.out = out;
    p.stream = s;
    return ATTN_OK;
}

int attn_sinks_prefill_window(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                              int total_q, int max_q_len, int max_seq_len, const void *q,
                              const void *k_cache, const void *v_cache,
                              const int32_t *block_table, const int32_t *seq_lens,
                              const int32_t *cu_seqlens_q, const float *sinks, float scale,
                              int window, void *out, void *stream)
{
    attn::PrefillLaunch p;
    bool empty = false;
    int rc = prepare_prefill(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                             num_pages, max_pages_per_seq, total_q, max_q_len, max_seq_len, q,
                             k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, sinks, scale,
                             window, out, stream, &p, &empty);
    if (rc != ATTN_OK || empty)
        return rc;
    if (dtype == ATTN_DTYPE_F32) {
        hipError_t e = attn::launch_rows_f32(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             max_pages_per_seq, total_q, q, k_cache, v_cache,
                                             block_table, seq_lens, cu_seqlens_q, sinks, scale,
                                             window, out, p.stream);
        return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
    }
    return attn::launch_prefill_bf16(p) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_sinks_mixed(int dtype, int num_decode_seqs, int num_prefill_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int page_size, int num_pages,
                     int max_pages_per_seq, int decode_max_seq_len, int total_q, int max_q_len,
                     int max_seq_len, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_table, const int32_t *seq_lens,
                     const int32_t *cu_seqlens_q, const float *sinks, float scale, void *out,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    const int nd = num_decode_seqs, np = num_prefill_seqs;
    if (nd < 0 || np < 0 || (long long)nd + np > 65535 || total_q < nd)
        return ATTN_ERR_SHAPE;
    // the decode part: sequences [0, nd), query rows 0 .. nd - 1
    attn::DecodeLaunch dp;
    int rc = prepare_decode(dtype, nd, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                            max_pages_per_seq, decode_max_seq_len, q, k_cache, v_cache,
                            block_table, seq_lens, sinks, scale, 0, out, workspace,
                            workspace_bytes, stream, true, true, &dp);
    if (rc != ATTN_OK)
        return rc;
    // the prefill part: sequences [nd, nd + np), their rows by cu_seqlens_q
    const size_t table_off = (size_t)nd * (size_t)max_pages_per_seq;
    const int32_t *bt_p = block_table ? block_table + table_off : nullptr;
    const int32_t *lens_p = seq_lens ? seq_lens + nd : nullptr;
    const int32_t *cu_p = cu_seqlens_q ? cu_seqlens_q + nd : nullptr;
    attn::PrefillLaunch pp;
    bool empty = false;
    rc = prepare_prefill(dtype, np, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                         max_pages_per_seq, total_q, max_q_len, max_seq_len, q, k_cache, v_cache,
                         bt_p, lens_p, cu_p, sinks, scale, 0, out, stream, &pp, &empty);
    if (rc != ATTN_OK)
        return rc;
    // one launch where the decode part takes the split pass and both parts
    // have work; otherwise (and for fp32) the two calls one after the other
    const bool fused = nd > 0 && !empty &&
                       decode_max_seq_len > attn::kDirectWindowMax && dp.num_wgs > 0 &&
                       !attn::debug_setting(attn::kDebugPrefillWaitAll);
    if (dtype == ATTN_DTYPE_F32) {
        // every row of the batch in one row-kernel launch: a decode row is a
        // one-row sequence there, computed as attn_sinks_decode computes it
        hipError_t e = attn::launch_rows_f32(nd + np, num_q_heads, num_kv_heads, head_dim,
                                             max_pages_per_seq, total_q, q, k_cache, v_cache,
                                             block_table, seq_lens, cu_seqlens_q, sinks, scale,
                                             0, out, reinterpret_cast<hipStream_t>(stream));
        return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
    }
    if (!fused) {
        // (the bf16 prefill addresses q and out by the absolute row offsets
        // in cu_seqlens_q, so the chunks' part of the arrays is theirs alone)
        if (nd > 0) {
            rc = attn_sinks_decode(dtype, nd, num_q_heads, num_kv_heads, head_dim, page_size,
                                   num_pages, max_pages_per_seq, decode_max_seq_len, q, k_cache,
                                   v_cache, block_table, seq_lens, sinks, scale, out, workspace,
                                   workspace_bytes, stream);
            if (rc != ATTN_OK)
                return rc;
        }
        if (empty)
            return ATTN_OK;
        return attn_sinks_prefill(dtype, np, num_q_heads, num_kv_heads, head_dim, page_size,
                                  num_pages, max_pages_per_seq, total_q, max_q_len, max_seq_len,
                                  q, k_cache, v_cache, bt_p, lens_p, cu_p, sinks, scale, out,
                                  stream);
    }
    if (attn::launch_mixed_bf16(dp, pp) != hipSuccess)
        return ATTN_ERR_HIP;
    return attn::launch_decode_merge(dp) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_sinks_append_kv(int dtype, int num_seqs, int num_kv_heads, int head_dim, int page_size,
                         int num_pages, int max_pages_per_seq, int max_seq_len, int total_new,
                         const void *k_new, const void *v_new, const int32_t *block_table,
                         const int32_t *seq_lens, const int32_t *cu_seqlens_new, void *k_cache,
                         void *v_cache, void *stream)
{
    int rc = check_append(dtype, num_seqs, num_kv_heads, head_dim, page_size, num_pages,
                          max_pages_per_seq, max_seq_len, total_new, k_new, v_new, block_table,
                          seq_lens, cu_seqlens_new, k_cache, v_cache);
    if (rc != ATTN_OK || num_seqs == 0 || total_new == 0)
        return rc;
    return attn::launch_append_kv(elem_bytes(dtype), num_seqs, num_kv_heads, head_dim,
                                  max_pages_per_seq, total_new, k_new, v_new, block_table,
                                  seq_lens, cu_seqlens_new, k_cache, v_cache,
                                  reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? ATTN_OK
               : ATTN_ERR_HIP;
}

int attn_sinks_rope_append(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                           int max_seq_len, int total_new, void *q, const void *k_new,
                           const void *v_new, const int32_t *positions, float rope_base,
                           float rope_scale, int orig_ctx, float beta_fast, float beta_slow,
                           const int32_t *block_table, const int32_t *seq_lens,
                           const int32_t *cu_seqlens_new, void *k_cache, void *v_cache,
                           void *stream)
{
    int rc = check_append(dtype, num_seqs, num_kv_heads, head_dim, page_size, num_pages,
                          max_pages_per_seq, max_seq_len, total_new, k_new, v_new, block_table,
                          seq_lens, cu_seqlens_new, k_cache, v_cache);
    if (rc != ATTN_OK)
        return rc;
    rc = check_common(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                      max_pages_per_seq, max_seq_len);
    if (rc != ATTN_OK)
        return rc;
    if (!(std::isfinite(rope_base) && rope_base > 0.f && rope_base != 1.f &&
          std::isfinite(rope_scale) && rope_scale > 0.f && orig_ctx > 0))
        return ATTN_ERR_SHAPE;
    if (rope_scale != 1.f && !(std::isfinite(beta_fast) && std::isfinite(beta_slow) &&
                               beta_fast > beta_slow && beta_slow > 0.f))
        return ATTN_ERR_SHAPE;
    if (num_seqs == 0 || total_new == 0)
        return ATTN_OK;
    if (!q || !positions)
        return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned4(positions))
        return ATTN_ERR_ALIGN;
    // YaRN frequencies: pair i turns at theta_i = base^(-2i/d).  The pair
    // that turns beta times within the original context sits at the
    // fractional index c(beta) = (d/2) ln(orig_ctx / (2 pi beta)) / ln(base);
    // pairs below c(beta_fast) keep theta_i, pairs above c(beta_slow) turn at
    // theta_i / scale, and the blend is linear in the pair index in between.
    // q and k are multiplied by 0.1 ln(scale) + 1.
    double freq[64];
    const double s = rope_scale;
    const double half = head_dim / 2.0, ln_base = std::log((double)rope_base);
    const double lo = half * std::log(orig_ctx / (2.0 * M_PI * beta_fast)) / ln_base;
    const double hi = half * std::log(orig_ctx / (2.0 * M_PI * beta_slow)) / ln_base;
    for (int i = 0; i < head_dim / 2; ++i) {
        const double theta = std::pow((double)rope_base, -2.0 * i / head_dim);
        if (s == 1.0) {
            freq[i] = theta;
            continue;
        }
        double ramp = (i - lo) / (hi - lo);
        ramp = ramp < 0.0 ? 0.0 : (ramp > 1.0 ? 1.0 : ramp);
        freq[i] = (1.0 - ramp) * theta + ramp * theta / s;
    }
    const float mscale = s > 1.0 ? (float)(0.1 * std::log(s) + 1.0) : 1.f;
    return attn::launch_rope_append(elem_bytes(dtype), num_seqs, num_q_heads, num_kv_heads,
                                    head_dim, max_pages_per_seq, total_new, q, k_new, v_new,
                                    positions, freq, mscale, block_table, seq_lens,
                                    cu_seqlens_new, k_cache, v_cache,
                                    reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? ATTN_OK
               : ATTN_ERR_HIP;
}

int attn_sinks_decode_append(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                             int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                             int max_seq_len, const void *q, const void *k_new,
                             const void *v_new, void *k_cache, void *v_cache,
                             const int32_t *block_table, const int32_t *seq_lens,
                             const float *sinks, float scale, int window, void *out,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    // every check of both steps runs before anything is enqueued
    attn::DecodeLaunch p;
    int rc = prepare_decode(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                            num_pages, max_pages_per_seq, max_seq_len, q, k_cache, v_cache,
                            block_table, seq_lens, sinks, scale, window, out, workspace,
                            workspace_bytes, stream, true, true, &p);
    if (rc != ATTN_OK || num_seqs == 0)
        return rc;
    rc = check_append(dtype, num_seqs, num_kv_heads, head_dim, page_size, num_pages,
                      max_pages_per_seq, max_seq_len, num_seqs, k_new, v_new, block_table,
                      seq_lens, nullptr, k_cache, v_cache);
    if (rc != ATTN_OK)
        return rc;
    if (attn::launch_append_kv(elem_bytes(dtype), num_seqs, num_kv_heads, head_dim,
                               max_pages_per_seq, num_seqs, k_new, v_new, block_table, seq_lens,
                               nullptr, k_cache, v_cache, p.stream) != hipSuccess)
        return ATTN_ERR_HIP;
    return attn_sinks_decode_window(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                    page_size, num_pages, max_pages_per_seq, max_seq_len, q,
                                    k_cache, v_cache, block_table, seq_lens, sinks, scale, window,
                                    out, workspace, workspace_bytes, stream);
}

int attn_sinks_prefill_append(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                              int total_q, int max_q_len, int max_seq_len, const void *q,
                              const void *k_new, const void *v_new, void *k_cache,
                              void *v_cache, const int32_t *block_table,
                              const int32_t *seq_lens, const int32_t *cu_seqlens_q,
                              const float *sinks, float scale, int window, void *out,
                              void *stream)
{
    // the prefill's own checks first (they enqueue nothing when they fail)
    int rc = check_common(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                          num_pages, max_pages_per_seq, max_seq_len);
    if (rc != ATTN_OK)
        return rc;
    if (total_q < 0 || max_q_len < 0 || max_q_len > max_seq_len || max_q_len > total_q ||
        !std::isfinite(scale) || window < 0)
        return ATTN_ERR_SHAPE;
    if (num_seqs == 0 || total_q == 0)
        return ATTN_OK;
    if (!q || !out || !cu_seqlens_q)
        return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned4(cu_seqlens_q) || (sinks && !aligned4(sinks)))
        return ATTN_ERR_ALIGN;
    rc = check_append(dtype, num_seqs, num_kv_heads, head_dim, page_size, num_pages,
                      max_pages_per_seq, max_seq_len, total_q, k_new, v_new, block_table,
                      seq_lens, cu_seqlens_q, k_cache, v_cache);
    if (rc != ATTN_OK)
        return rc;
    if (attn::launch_append_kv(elem_bytes(dtype), num_seqs, num_kv_heads, head_dim,
                               max_pages_per_seq, total_q, k_new, v_new, block_table, seq_lens,
                               cu_seqlens_q, k_cache, v_cache,
                               reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return ATTN_ERR_HIP;
    return attn_sinks_prefill_window(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                     page_size, num_pages, max_pages_per_seq, total_q, max_q_len,
                                     max_seq_len, q, k_cache, v_cache, block_table, seq_lens,
                                     cu_seqlens_q, sinks, scale, window, out, stream);
}

size_t attn_sinks_decode_multi_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                               int head_dim, int max_seq_len, int max_q_len)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
        max_q_len < 0 || !supported_head_dim(head_dim) || num_q_heads % num_kv_heads != 0 ||
        num_q_heads / num_kv_heads > kMaxGroup)
        return 0;
    if (!multi_packed(num_q_heads / num_kv_heads, max_q_len))
        return 0;  // such calls run the prefill kernel, which needs no scratch
    return decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, nullptr,
                            nullptr, max_q_len);
}

int attn_sinks_decode_multi(int dtype, int num_seqs, int num_q_heads, int num_kv_heads,
                            int head_dim, int page_size, int num_pages, int max_pages_per_seq,
                            int total_q, int max_q_len, int max_seq_len, const void *q,
                            const void *k_cache, const void *v_cache, const int32_t *block_table,
                            const int32_t *seq_lens, const int32_t *cu_seqlens_q,
                            const float *sinks, float scale, void *out, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    const bool packed = dtype == ATTN_DTYPE_BF16 &&
                        multi_packed(num_kv_heads > 0 ? num_q_heads / num_kv_heads : 0, max_q_len);
    if (!packed)  // fp32, or more packed rows than the split pass takes
        return attn_sinks_prefill(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  page_size, num_pages, max_pages_per_seq, total_q, max_q_len,
                                  max_seq_len, q, k_cache, v_cache, block_table, seq_lens,
                                  cu_seqlens_q, sinks, scale, out, stream);
    attn::DecodeLaunch p;
    int rc = prepare_decode(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                            num_pages, max_pages_per_seq, max_seq_len, q, k_cache, v_cache,
                            block_table, seq_lens, sinks, scale, 0, out, workspace,
                            workspace_bytes, stream, true, true, &p);
    if (rc != ATTN_OK)
        return rc;
    if (total_q < 0 || max_q_len < 0 || max_q_len > max_seq_len || max_q_len > total_q)
        return ATTN_ERR_SHAPE;
    if (num_seqs == 0 || total_q == 0)
        return ATTN_OK;
    if (!cu_seqlens_q)
        return ATTN_ERR_NULL;
    if (!aligned4(cu_seqlens_q) || (workspace && !aligned16(workspace)))
        return ATTN_ERR_ALIGN;
    size_t acc_offset = 0;
    const size_t need = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                         max_seq_len, nullptr, &acc_offset, max_q_len);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return workspace ? ATTN_ERR_WORKSPACE : ATTN_ERR_NULL;
    p.cu_seqlens_q = cu_seqlens_q;
    p.q_max = max_q_len;
    float *ws = static_cast<float *>(workspace);
    p.part_ml = ws;
    p.part_acc = ws ? ws + acc_offset : nullptr;
    if (attn::launch_decode_split_bf16(p) != hipSuccess)
        return ATTN_ERR_HIP;
    return attn::launch_decode_merge(p) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_sinks_ragged(int dtype, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int total_q, int total_kv, int max_q_len, int max_kv_len, int causal,
                      const void *q, const void *k, const void *v, const int32_t *cu_seqlens_q,
                      const int32_t *cu_seqlens_kv, const float *sinks, float scale, void *out,
                      float *lse, void *stream)
{
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16)
        return ATTN_ERR_UNSUPPORTED;
    if (dtype != ATTN_DTYPE_BF16 || !supported_head_dim(head_dim))
        return ATTN_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || total_q < 0 || total_kv < 0 ||
        max_q_len < 0 || max_kv_len < 0 || max_q_len > total_q || max_kv_len > total_kv ||
        (causal != 0 && causal != 1) || num_q_heads % num_kv_heads != 0)
        return ATTN_ERR_SHAPE;
    if (num_q_heads / num_kv_heads > kMaxGroup)
        return ATTN_ERR_UNSUPPORTED;
    if (causal && max_q_len > max_kv_len)
        return ATTN_ERR_SHAPE;
    if (num_seqs > 65535 || num_q_heads > 65535)
        return ATTN_ERR_SHAPE;
    // the per-lane byte offsets of a sequence's K/V rows must fit 31 bits
    if ((long long)max_kv_len * num_kv_heads * head_dim * 2 >= (1LL << 31))
        return ATTN_ERR_SHAPE;
    if (!std::isfinite(scale))
        return ATTN_ERR_SHAPE;
    if (num_seqs == 0 || total_q == 0)
        return ATTN_OK;
    if (!q || !out || !cu_seqlens_q || !cu_seqlens_kv || (total_kv > 0 && (!k || !v)))
        return ATTN_ERR_NULL;
    const void *vec[] = {q, k, v, out};
    for (const void *ptr : vec)
        if (ptr && !aligned16(ptr))
            return ATTN_ERR_ALIGN;
    const void *words[] = {cu_seqlens_q, cu_seqlens_kv, sinks, lse};
    for (const void *ptr : words)
        if (ptr && !aligned4(ptr))
            return ATTN_ERR_ALIGN;
    attn::PrefillLaunch p;
    p.dtype = dtype;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.head_dim = head_dim;
    p.max_pages_per_seq = 0;
    p.total_q = total_q;
    p.max_q_len = max_q_len;
    p.max_seq_len = max_kv_len;
    p.window = 0;
    p.cu_seqlens_kv = cu_seqlens_kv;
    p.causal = causal;
    p.lse = lse;
    p.q = q;
    p.k_cache = k;
    p.v_cache = v;
    p.block_table = nullptr;
    p.seq_lens = nullptr;
    p.cu_seqlens_q = cu_seqlens_q;
    p.sinks = sinks;
    p.scale = scale;
    p.out = out;
    p.stream = reinterpret_cast<hipStream_t>(stream);
    return attn::launch_prefill_bf16(p) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

const char *attn_sinks_status_string(int status)
{
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case ATTN_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, page_size or group size";
    case ATTN_ERR_WORKSPACE: return "decode workspace is smaller than required";
    case ATTN_ERR_ALIGN: return "a pointer is not aligned as required";
    case ATTN_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case ATTN_ERR_SCRATCH:
        return "the call needs more than the 32 MiB fixed scratch of attn_sinks_decode_noalloc "
               "(attn_sinks_decode_workspace_bytes gives the size it needs)";
    default: return "unknown status";
    }
}

int attn_sinks_version(void) { return kVersion; }

int attn_sinks_set_debug(int setting, int value)
{
    if (setting < 0 || setting >= attn::kDebugSettings)
        return -1;
    debug_init();
    return g_debug[setting].exchange(value != 0 ? 1 : 0);
}

}  // extern "C"
