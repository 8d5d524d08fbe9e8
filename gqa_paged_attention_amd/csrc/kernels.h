// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct DecodeLaunch {
    int dtype;  // 0 f32, 1 bf16
    int num_seqs, num_q_heads, num_kv_heads, head_dim;
    int max_pages_per_seq;
    int num_wgs;        // split-pass workgroups per KV-head group
    int heads_per_wg;   // KV heads (one wave each) per split-pass workgroup
    int window;         // sliding window W (keys L - W .. L - 1), 0: none
    // multi-token decode: query offsets [num_seqs + 1] (NULL: one token per
    // sequence) and the largest number of query tokens of a sequence
    const int32_t *cu_seqlens_q;
    int q_max;
    const void *q, *k_cache, *v_cache;
    const int32_t *block_table, *seq_lens;
    const float *sinks;
    float scale;
    void *out;
    float *part_ml;     // [slots][q_max][Hq][2],   slots = num_seqs + num_wgs
    float *part_acc;    // [slots][q_max][Hq][head_dim]
    hipStream_t stream;
};

struct PrefillLaunch {
    int dtype;
    int num_seqs, num_q_heads, num_kv_heads, head_dim;
    int max_pages_per_seq, total_q, max_q_len, max_seq_len;
    int window;         // sliding window W (keys p - W + 1 .. p), 0: none
    // ragged cache-free attention: K/V rows [tokens][Hkv][d] at offsets
    // cu_seqlens_kv [num_seqs + 1] (NULL: the paged cache and block_table)
    const int32_t *cu_seqlens_kv;
    int causal;         // 0: every row sees all keys of its sequence
    float *lse;         // [total_q][Hq] natural-log LSE (sink included), or NULL
    const void *q, *k_cache, *v_cache;
    const int32_t *block_table, *seq_lens, *cu_seqlens_q;
    const float *sinks;
    float scale;
    void *out;
    hipStream_t stream;
};

// Debug settings (attn_sinks_set_debug; environment defaults read once):
// kDebugPrefillOneHead gives every prefill workgroup one query head where it
// would take four (ATTN_SINKS_PREFILL_ONE_HEAD=1), kDebugPrefillWaitAll makes
// the prefill tile waits take every load in flight
// (ATTN_SINKS_PREFILL_WAIT_ALL=1), kDebugPrefillWindowStreamed runs the
// windowed prefill in the kernel whose waves stream their own blocks
// (ATTN_SINKS_PREFILL_WINDOW_STREAMED=1).  Every setting gives results within
// the same bar (the first two the same bits).
constexpr int kDebugPrefillOneHead = 0;
constexpr int kDebugPrefillWaitAll = 1;
constexpr int kDebugPrefillWindowStreamed = 2;
constexpr int kDebugSettings = 3;
int debug_setting(int id);

// The most packed query rows (G times query tokens per sequence) the
// multi-token decode takes per KV head (in layers of up to 64 rows at d = 64
// and of 32 at d = 128); beyond that the prefill kernel runs.
constexpr int kMultiRowsMax = 128;

// Decode split pass: up to 4 KV heads (waves) per workgroup; the grid gives
// every one of MI355X's 256 CUs the same number of workgroups, with at least
// 4 waves per CU.
constexpr int kDecodeMaxHeadsPerWg = 4;
constexpr int kDeviceCUs = 256;
constexpr int kDecodeMinWavesPerCU = 4;

// Split pass: partial (max, sum, weighted values) per split into the workspace.
hipError_t launch_decode_split_bf16(const DecodeLaunch &p);
// Merge pass: combine the splits of each (sequence, head), fold the sink,
// write out in p.dtype.
hipError_t launch_decode_merge(const DecodeLaunch &p);
// Direct decode (bf16, one query token, 0 < window <= kDirectWindowMax and
// window < the length bound, or a length bound <= kDirectWindowMax): one wave
// per (sequence, KV head) over the visible keys, sink folded, output
// written; no workspace, no merge.
constexpr int kDirectWindowMax = 512;
hipError_t launch_decode_direct_bf16(const DecodeLaunch &p);
hipError_t launch_prefill_bf16(const PrefillLaunch &p);
// The split pass of a single-token decode batch (d) and the causal prefill of
// chunks (p) in one launch, the split workgroups first; the caller then runs
// launch_decode_merge(d).  Both on p.stream; same results as the two kernels.
hipError_t launch_mixed_bf16(const DecodeLaunch &d, const PrefillLaunch &p);
// KV append: new rows [total_new][Hkv][d] into their page slots (f32 or bf16,
// elem_bytes 4 or 2); cu_seqlens_new NULL means one new token per sequence.
hipError_t launch_append_kv(int elem_bytes, int num_seqs, int num_kv_heads, int head_dim,
                            int max_pages_per_seq, int total_new, const void *k_new,
                            const void *v_new, const int32_t *block_table,
                            const int32_t *seq_lens, const int32_t *cu_seqlens_new,
                            void *k_cache, void *v_cache, hipStream_t stream);
// Rotary embedding (per-pair frequencies freq[head_dim / 2], factor mscale)
// of q in place and of the new K rows into their cache slots, V appended.
hipError_t launch_rope_append(int elem_bytes, int num_seqs, int num_q_heads, int num_kv_heads,
                              int head_dim, int max_pages_per_seq, int total_new, void *q,
                              const void *k_new, const void *v_new, const int32_t *positions,
                              const double *freq, float mscale, const int32_t *block_table,
                              const int32_t *seq_lens, const int32_t *cu_seqlens_new,
                              void *k_cache, void *v_cache, hipStream_t stream);
// fp32 path (full rows, no split), used for both decode and prefill.
hipError_t launch_rows_f32(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int max_pages_per_seq, int total_q, const void *q,
                           const void *k_cache, const void *v_cache, const int32_t *block_table,
                           const int32_t *seq_lens, const int32_t *cu_seqlens_q,
                           const float *sinks, float scale, int window, void *out,
                           hipStream_t stream);

}  // namespace attn
