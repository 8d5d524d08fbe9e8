// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer around the library's host code (tests/
// test_sanitizers.py builds and runs it on the CPU).  Every call below either
// fails the host checks or has nothing to enqueue, so no call reaches the HIP
// runtime; pointers are stand-in addresses that are never dereferenced.
// Prints one line per failed expectation and exits nonzero if there was any.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn_sinks.h"

namespace {

int failures = 0;

void expect(const char *what, int got, int want)
{
    if (got != want) {
        std::printf("FAIL %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

void *at(uintptr_t a) { return reinterpret_cast<void *>(a); }
const int32_t *ip(uintptr_t a) { return reinterpret_cast<const int32_t *>(a); }
const float *fp(uintptr_t a) { return reinterpret_cast<const float *>(a); }

constexpr uintptr_t F = 0x10000;  // 16-byte aligned, non-null
const float kNan = std::nanf("");

int decode(int dtype, int B, int Hq, int Hkv, int d, int P, int max_len, uintptr_t q,
           uintptr_t out, uintptr_t ws, size_t ws_bytes, float scale)
{
    return attn_sinks_decode(dtype, B, Hq, Hkv, d, P, 8, 4, max_len, at(q), at(F), at(F), ip(F),
                             ip(F), nullptr, scale, at(out), at(ws), ws_bytes, nullptr);
}

int prefill(int dtype, int B, int Hq, int Hkv, int d, int total_q, int max_q, int max_len,
            uintptr_t cu, uintptr_t out, float scale, int window)
{
    return attn_sinks_prefill_window(dtype, B, Hq, Hkv, d, 16, 8, 4, total_q, max_q, max_len,
                                     at(F), at(F), at(F), ip(F), ip(F), ip(cu), nullptr, scale,
                                     window, at(out), nullptr);
}

}  // namespace

int main()
{
    const size_t big = (size_t)1 << 30;
    expect("decode dtype", decode(2, 2, 8, 2, 64, 16, 64, F, F, F, big, .125f),
           ATTN_ERR_UNSUPPORTED);
    expect("decode head_dim", decode(1, 2, 8, 2, 96, 16, 64, F, F, F, big, .125f),
           ATTN_ERR_UNSUPPORTED);
    expect("decode page", decode(1, 2, 8, 2, 64, 32, 64, F, F, F, big, .125f),
           ATTN_ERR_UNSUPPORTED);
    expect("decode group", decode(1, 2, 8, 3, 64, 16, 64, F, F, F, big, .125f), ATTN_ERR_SHAPE);
    expect("decode length bound", decode(1, 2, 8, 2, 64, 16, 65, F, F, F, big, .125f),
           ATTN_ERR_SHAPE);
    expect("decode scale", decode(1, 2, 8, 2, 64, 16, 64, F, F, F, big, kNan), ATTN_ERR_SHAPE);
    expect("decode q", decode(1, 2, 8, 2, 64, 16, 64, 0, F, F, big, .125f), ATTN_ERR_NULL);
    expect("decode workspace", decode(1, 2, 8, 2, 64, 16, 64, F, F, F, 16, .125f),
           ATTN_ERR_WORKSPACE);
    expect("decode align", decode(1, 2, 8, 2, 64, 16, 64, F + 8, F, F, big, .125f),
           ATTN_ERR_ALIGN);
    expect("decode empty", decode(1, 0, 8, 2, 64, 16, 64, F, F, F, big, .125f), ATTN_OK);
    expect("decode window", attn_sinks_decode_window(1, 2, 8, 2, 64, 16, 8, 4, 64, at(F), at(F),
                                                     at(F), ip(F), ip(F), nullptr, .125f, -1,
                                                     at(F), at(F), big, nullptr),
           ATTN_ERR_SHAPE);
    expect("noalloc beyond the scratch",
           attn_sinks_decode_noalloc(1, 2000, 64, 8, 64, 16, 1, 512, 8192, at(F), at(F), at(F),
                                     ip(F), ip(F), nullptr, .125f, 0, at(F), nullptr),
           ATTN_ERR_SCRATCH);
    expect("noalloc window", attn_sinks_decode_noalloc(1, 2, 8, 2, 64, 16, 8, 4, 64, at(F),
                                                       at(F), at(F), ip(F), ip(F), nullptr,
                                                       .125f, -1, at(F), nullptr),
           ATTN_ERR_SHAPE);
    expect("noalloc empty", attn_sinks_decode_noalloc(1, 0, 8, 2, 64, 16, 8, 4, 64, at(F), at(F),
                                                      at(F), ip(F), ip(F), nullptr, .125f, 0,
                                                      at(F), nullptr),
           ATTN_OK);
    expect("partials dtype", attn_sinks_decode_partials(0, 2, 8, 2, 64, 16, 8, 4, 64, at(F),
                                                        at(F), at(F), ip(F), ip(F), .125f, at(F),
                                                        big, nullptr),
           ATTN_ERR_UNSUPPORTED);
    expect("merge workspace", attn_sinks_decode_merge(1, 2, 8, 2, 64, 64, ip(F), nullptr, at(F),
                                                      16, at(F), nullptr),
           ATTN_ERR_WORKSPACE);
    expect("prefill q rows", prefill(1, 2, 8, 2, 64, 40, 41, 64, F, F, .125f, 0),
           ATTN_ERR_SHAPE);
    expect("prefill cu", prefill(1, 2, 8, 2, 64, 40, 32, 64, 0, F, .125f, 0), ATTN_ERR_NULL);
    expect("prefill align", prefill(1, 2, 8, 2, 64, 40, 32, 64, F + 2, F, .125f, 0),
           ATTN_ERR_ALIGN);
    expect("prefill window", prefill(1, 2, 8, 2, 64, 40, 32, 64, F, F, .125f, -3),
           ATTN_ERR_SHAPE);
    expect("prefill empty", prefill(1, 2, 8, 2, 64, 0, 0, 64, F, F, .125f, 0), ATTN_OK);
    expect("append one token each",
           attn_sinks_append_kv(1, 2, 2, 64, 16, 8, 4, 64, 5, at(F), at(F), ip(F), ip(F),
                                nullptr, at(F), at(F), nullptr),
           ATTN_ERR_SHAPE);
    expect("append null", attn_sinks_append_kv(1, 2, 2, 64, 16, 8, 4, 64, 2, nullptr, at(F),
                                               ip(F), ip(F), nullptr, at(F), at(F), nullptr),
           ATTN_ERR_NULL);
    expect("rope base", attn_sinks_rope_append(1, 2, 8, 2, 64, 16, 8, 4, 64, 5, at(F), at(F),
                                               at(F), ip(F), 1.f, 32.f, 4096, 32.f, 1.f, ip(F),
                                               ip(F), ip(F), at(F), at(F), nullptr),
           ATTN_ERR_SHAPE);
    expect("rope betas", attn_sinks_rope_append(1, 2, 8, 2, 64, 16, 8, 4, 64, 5, at(F), at(F),
                                                at(F), ip(F), 1e4f, 32.f, 4096, 1.f, 1.f,
                                                ip(F), ip(F), ip(F), at(F), at(F), nullptr),
           ATTN_ERR_SHAPE);
    expect("decode_append workspace",
           attn_sinks_decode_append(1, 2, 8, 2, 64, 16, 8, 4, 64, at(F), at(F), at(F), at(F),
                                    at(F), ip(F), ip(F), nullptr, .125f, 0, at(F), at(F), 16,
                                    nullptr),
           ATTN_ERR_WORKSPACE);
    expect("prefill_append align",
           attn_sinks_prefill_append(1, 2, 8, 2, 64, 16, 8, 4, 40, 32, 64, at(F), at(F + 4),
                                     at(F), at(F), at(F), ip(F), ip(F), ip(F), nullptr, .125f, 0,
                                     at(F), nullptr),
           ATTN_ERR_ALIGN);
    expect("multi cu", attn_sinks_decode_multi(1, 2, 8, 2, 64, 16, 8, 4, 8, 4, 64, at(F), at(F),
                                               at(F), ip(F), ip(F), nullptr, nullptr, .125f,
                                               at(F), at(F), big, nullptr),
           ATTN_ERR_NULL);
    expect("ragged causal rows", attn_sinks_ragged(1, 2, 8, 2, 64, 40, 40, 33, 32, 1, at(F),
                                                   at(F), at(F), ip(F), ip(F), nullptr, .125f,
                                                   at(F), nullptr, nullptr),
           ATTN_ERR_SHAPE);
    expect("ragged fp32", attn_sinks_ragged(0, 2, 8, 2, 64, 40, 40, 32, 32, 1, at(F), at(F),
                                            at(F), ip(F), ip(F), nullptr, .125f, at(F), nullptr,
                                            nullptr),
           ATTN_ERR_UNSUPPORTED);
    expect("workspace bytes, bad group",
           (int)attn_sinks_decode_workspace_bytes(64, 64, 7, 64, 8192), 0);
    expect("multi workspace bytes, bad dim",
           (int)attn_sinks_decode_multi_workspace_bytes(64, 64, 8, 80, 8192, 4), 0);
    for (int s = -2; s < 12; ++s)
        if (!attn_sinks_status_string(s) || !std::strlen(attn_sinks_status_string(s)))
            expect("status string", s, -100);
    expect("version", attn_sinks_version() >= 100, 1);
    std::printf("%s: %d failed\n", failures ? "FAIL" : "ok", failures);
    return failures ? 1 : 0;
}
