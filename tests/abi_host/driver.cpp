// Drives every entry point of the C ABI with invalid and extreme arguments
// (and with valid ones, which end in a device, allocation or launch status
// since the launchers are stubs); exits non-zero on an unexpected status.
// Built host-only with the address and undefined-behaviour sanitizers, so any
// out-of-bounds access, overflow or other undefined behaviour in the argument
// checks aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "fa.h"

namespace {

int failures = 0, checks = 0;

void expect(fa_status got, fa_status want, const char* what) {
    ++checks;
    if (got != want) {
        std::printf("FAIL %s: status %d, want %d\n", what, static_cast<int>(got), static_cast<int>(want));
        ++failures;
    }
}

void expect_not_ok(fa_status got, const char* what) {
    ++checks;
    if (got == FA_OK) {
        std::printf("FAIL %s: FA_OK from stub launchers\n", what);
        ++failures;
    }
}

void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

}  // namespace

int main() {
    const int64_t kMax = std::numeric_limits<int64_t>::max(), kMin = std::numeric_limits<int64_t>::min();
    const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();
    void *q = P(0x10000), *k = P(0x20000), *v = P(0x30000), *o = P(0x40000);
    float* lse = static_cast<float*>(P(0x50000));

    ++checks;
    if (fa_abi_version() != FA_ABI_VERSION) ++failures;
    for (int s : {0, 5, 11, 12, 999, -1, 0x7FFFFFFF}) {
        const char* t = fa_status_string(static_cast<fa_status>(s));
        ++checks;
        if (t == nullptr || std::strlen(t) == 0) ++failures;
    }

    // fa_fwd: every validation branch, extreme shapes (no overflow allowed)
    expect(fa_fwd(nullptr, k, v, o, lse, 1, 1, 64, 64, 0, 0.1f, FA_BF16, nullptr), FA_ERR_NULL_POINTER, "fwd null");
    const int64_t shapes[][4] = {{0, 1, 64, 64}, {1, 0, 64, 64}, {1, 1, 0, 64}, {1, 1, 64, 0},
                                 {kMax, kMax, kMax, 128}, {1, 1, kMax, 64}, {kMax, 1, 1, 32}, {1, kMax, 64, 64},
                                 {kMin, 1, 64, 64}, {1, 1, kMin, 64}, {1, 1, 64, kMin}, {65536, 65536, 64, 64},
                                 {1, 1, (int64_t{1} << 31), 32}};
    for (const auto& sh : shapes)
        expect(fa_fwd(q, k, v, o, lse, sh[0], sh[1], sh[2], sh[3], 0, 0.1f, FA_BF16, nullptr), FA_ERR_INVALID_SHAPE,
               "fwd shape");
    expect(fa_fwd(q, k, v, o, lse, 1, 1, 64, 48, 0, 0.1f, FA_BF16, nullptr), FA_ERR_UNSUPPORTED_HEAD_DIM, "fwd d=48");
    expect(fa_fwd(q, k, v, o, lse, 1, 1, 64, kMax, 0, 0.1f, FA_BF16, nullptr), FA_ERR_UNSUPPORTED_HEAD_DIM, "fwd d=max");
    for (float sc : {nan, inf, -inf, 0.0f, -1.0f, -0.0f})
        expect(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, 0, sc, FA_BF16, nullptr), FA_ERR_INVALID_SCALE, "fwd scale");
    for (int dt : {4, 7, -1, 0x7FFFFFFF, -0x7FFFFFFF - 1})
        expect(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, 0, 0.1f, static_cast<fa_dtype>(dt), nullptr),
               FA_ERR_INVALID_DTYPE, "fwd dtype");
    expect(fa_bwd(q, k, v, o, P(0x100000), lse, P(0xD0000), P(0xE0000), P(0xF0000), 1, 2, 64, 128, 1, 0.1f,
                  static_cast<fa_dtype>(-5), nullptr),
           FA_ERR_INVALID_DTYPE, "bwd dtype");
    expect(fa_fwd(q, k, v, o, lse, 1, 1, 64, 64, 2, 0.1f, FA_BF16, nullptr), FA_ERR_INVALID_ARGUMENT, "fwd causal");
    expect(fa_fwd(q, k, v, q, lse, 1, 1, 64, 64, 0, 0.1f, FA_BF16, nullptr), FA_ERR_INVALID_ARGUMENT, "fwd alias");
    expect(fa_fwd(P(0x10002), k, v, o, lse, 1, 1, 64, 64, 0, 0.1f, FA_BF16, nullptr), FA_ERR_MISALIGNED, "fwd align");
    expect(fa_fwd(q, k, v, o, static_cast<float*>(P(0x50002)), 1, 1, 64, 64, 0, 0.1f, FA_BF16, nullptr),
           FA_ERR_MISALIGNED, "fwd lse align");
    for (int dt = 0; dt < 4; ++dt)
        for (int64_t d : {32, 64, 128})
            expect_not_ok(fa_fwd(q, k, v, o, lse, 2, 3, 1000, d, dt & 1, 0.1f, static_cast<fa_dtype>(dt), nullptr),
                          "fwd valid");
    expect_not_ok(fa_fwd(q, k, v, o, nullptr, 1, 1, 1, 128, 1, 0.1f, FA_BF16, nullptr), "fwd no lse");

    // quantisers and the FP8 forward
    uint8_t *q8 = static_cast<uint8_t*>(P(0x60000)), *k8 = static_cast<uint8_t*>(P(0x70000));
    float *qs = static_cast<float*>(P(0x80000)), *ks = static_cast<float*>(P(0x90000));
    expect(fa_quant_fp8_e4m3(nullptr, q8, qs, 1, 64, 64, nullptr), FA_ERR_NULL_POINTER, "quant null");
    expect(fa_quant_fp8_e4m3(q, q8, qs, kMax, kMax, 64, nullptr), FA_ERR_INVALID_SHAPE, "quant shape");
    expect_not_ok(fa_quant_fp8_e4m3(q, q8, qs, 4, 100, 64, nullptr), "quant valid");
    expect(fa_quant_v_pow2(v, q8, k8, kMin, 64, 64, nullptr), FA_ERR_INVALID_SHAPE, "quant_v shape");
    expect_not_ok(fa_quant_v_pow2(v, q8, k8, 4, 100, 128, nullptr), "quant_v valid");
    expect(fa_fwd_fp8(q8, qs, k8, ks, v, o, lse, 1, 1, kMax, 128, 1, 0.1f, nullptr), FA_ERR_INVALID_SHAPE, "fp8 shape");
    expect(fa_fwd_fp8(q8, qs, k8, ks, v, o, lse, 1, 1, 64, 128, 1, nan, nullptr), FA_ERR_INVALID_SCALE, "fp8 scale");
    expect_not_ok(fa_fwd_fp8(q8, qs, k8, ks, v, o, lse, 1, 2, 300, 128, 1, 0.1f, nullptr), "fp8 valid");

    // key ranges, merge, split-KV
    float *op = static_cast<float*>(P(0xA0000)), *lp = static_cast<float*>(P(0xB0000));
    const int64_t ranges[][2] = {{-64, 64}, {128, 64}, {0, 1001}, {1, 64}, {0, 65}, {kMin, kMax}, {kMax, kMax}};
    for (const auto& r : ranges)
        expect(fa_fwd_partial(q, k, v, op, lp, 1, 2, 1000, 64, r[0], r[1], 1, 0.1f, nullptr), FA_ERR_INVALID_ARGUMENT,
               "partial range");
    expect_not_ok(fa_fwd_partial(q, k, v, op, lp, 1, 2, 1000, 64, 64, 1000, 1, 0.1f, nullptr), "partial valid");
    for (int64_t n : {int64_t{0}, int64_t{1025}, kMax, kMin})
        expect(fa_merge(op, lp, n, o, lse, 1, 2, 100, 64, nullptr), FA_ERR_INVALID_ARGUMENT, "merge parts");
    expect_not_ok(fa_merge(op, lp, 4, o, lse, 1, 2, 100, 64, nullptr), "merge valid");
    for (int64_t n : {int64_t{0}, int64_t{1025}, kMax, kMin})
        expect(fa_fwd_splitkv(q, k, v, o, lse, 1, 2, 1000, 128, 1, 0.1f, n, nullptr), FA_ERR_INVALID_ARGUMENT,
               "splitkv splits");
    expect_not_ok(fa_fwd_splitkv(q, k, v, o, lse, 1, 2, 1000, 128, 1, 0.1f, 3, nullptr), "splitkv valid");
    for (int64_t n : {int64_t{0}, int64_t{1025}, kMax, kMin})
        expect(fa_fwd_splitkv_noalloc(q, k, v, o, lse, 1, 2, 1000, 128, 1, 0.1f, n, nullptr), FA_ERR_INVALID_ARGUMENT,
               "splitkv_noalloc splits");
    expect(fa_fwd_splitkv_noalloc(q, k, v, o, lse, kMax, kMax, 1000, 128, 1, 0.1f, 2, nullptr), FA_ERR_INVALID_SHAPE,
           "splitkv_noalloc shape");
    // 2 x 4 x 16384 x (128 + 1) x 4 bytes fit the 128 MiB buffer; 3 x 8 x 16384 ... do not
    expect(fa_fwd_splitkv_noalloc(q, k, v, o, lse, 1, 8, 16384, 128, 1, 0.1f, 3, nullptr), FA_ERR_SCRATCH_LIMIT,
           "splitkv_noalloc limit");
    expect(fa_fwd_splitkv_noalloc(q, k, v, o, lse, 1, 1, 1 << 20, 128, 1, 0.1f, 1024, nullptr), FA_ERR_SCRATCH_LIMIT,
           "splitkv_noalloc limit, many splits");
    expect_not_ok(fa_fwd_splitkv_noalloc(q, k, v, o, lse, 1, 4, 16384, 128, 1, 0.1f, 2, nullptr),
                  "splitkv_noalloc valid");

    // block-sparse
    const uint8_t* mask = static_cast<const uint8_t*>(P(0xC0000));
    for (int64_t st : {int64_t{1}, int64_t{-1}, kMax, kMin})
        expect(fa_fwd_blocksparse(q, k, v, o, lse, 1, 2, 1000, 64, mask, st, 1, 0.1f, nullptr), FA_ERR_INVALID_ARGUMENT,
               "blocksparse stride");
    expect(fa_fwd_blocksparse(q, k, v, o, lse, 1, 2, 1000, 64, nullptr, 0, 1, 0.1f, nullptr), FA_ERR_NULL_POINTER,
           "blocksparse null");
    expect_not_ok(fa_fwd_blocksparse(q, k, v, o, lse, 1, 2, 1000, 64, mask, 16 * 16, 1, 0.1f, nullptr),
                  "blocksparse valid");

    // backward
    void *dq = P(0xD0000), *dk = P(0xE0000), *dv = P(0xF0000), *dout = P(0x100000);
    expect(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, kMax, 2, 64, 128, 1, 0.1f, FA_BF16, nullptr), FA_ERR_INVALID_SHAPE,
           "bwd shape");
    expect(fa_bwd(q, k, v, o, dout, nullptr, dq, dk, dv, 1, 2, 64, 128, 1, 0.1f, FA_BF16, nullptr), FA_ERR_NULL_POINTER,
           "bwd null lse");
    expect(fa_bwd(q, k, v, o, dout, lse, q, dk, dv, 1, 2, 64, 128, 1, 0.1f, FA_BF16, nullptr), FA_ERR_INVALID_ARGUMENT,
           "bwd alias");
    expect_not_ok(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, 1, 2, 300, 128, 1, 0.1f, FA_BF16, nullptr), "bwd valid");

    std::printf("%d checks, %d failures\n", checks, failures);
    return failures == 0 ? 0 : 1;
}
