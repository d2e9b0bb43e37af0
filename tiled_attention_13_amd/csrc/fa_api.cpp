// C ABI of the attention library (declared in include/fa.h): forward in four
// element types, partial / merged / split-KV and block-sparse forwards, FP8
// pre-passes, and the backward.
//
// Every argument is checked before the first HIP call, so argument errors come
// back synchronously and can be exercised on a machine without a GPU.  After
// validation the call checks (once per device) that it runs on gfx950 and
// enqueues the kernels on the caller's stream.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "fa_internal.h"
#include "fa_scratch.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxParts = 1024;     // partial results per merge / splits per call
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_state[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

fa_status check_shape(int64_t B, int64_t H, int64_t N, int64_t d) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_SHAPE;
    if (d != 32 && d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    // element offsets inside a launch are formed in 32-bit arithmetic per (b, h)
    // slice and 64-bit across slices; keep the whole tensor, with N rounded up
    // to the 64-key tile (the transposed workspaces), below 2^31 elements
    const long double np = std::ceil(static_cast<long double>(N) / 64.0L) * 64.0L;   // exact for any int64 N
    const long double total = static_cast<long double>(B) * H * np * d;
    if (total >= 2147483648.0L) return FA_ERR_INVALID_SHAPE;
    return FA_OK;
}

fa_status check_scale(float s) {
    if (!std::isfinite(s) || !(s > 0.0f)) return FA_ERR_INVALID_SCALE;
    return FA_OK;
}

fa_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED_ARCH;
    int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_HIP;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? FA_OK : FA_ERR_UNSUPPORTED_ARCH;
}

fa_status launch_status(hipError_t e) {
    if (e == hipSuccess) return FA_OK;
    if (e == hipErrorOutOfMemory) return FA_ERR_OUT_OF_MEMORY;
    return FA_ERR_LAUNCH;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int padded_keys(int n) { return (n + fa::kKeyTile - 1) / fa::kKeyTile * fa::kKeyTile; }

// bytes of a transposed copy [BH, d, N rounded up to a key tile] bf16 (backward workspaces)
size_t vt_bytes(int BH, int n, int d) { return static_cast<size_t>(BH) * d * padded_keys(n) * 2; }

// Stream-ordered workspace; a request of zero bytes allocates nothing.  With
// FA_TEST_FAIL_ALLOC=1 in the environment (read at each call) every request
// fails as an exhausted device would, so tests can reach the out-of-memory path.
fa_status ws_alloc(void** p, size_t bytes, hipStream_t s) {
    *p = nullptr;
    if (bytes == 0) return FA_OK;
    const char* fail = std::getenv("FA_TEST_FAIL_ALLOC");
    if (fail != nullptr && fail[0] == '1') return FA_ERR_OUT_OF_MEMORY;
    if (hipMallocAsync(p, bytes, s) != hipSuccess || *p == nullptr) {
        (void)hipGetLastError();
        *p = nullptr;
        return FA_ERR_OUT_OF_MEMORY;
    }
    return FA_OK;
}

hipError_t ws_free(void* p, hipStream_t s) { return p ? hipFreeAsync(p, s) : hipSuccess; }

// Split-KV: argument checks shared by both entry points, the byte layout of
// the partial results, and the launches on a caller-provided buffer.
fa_status splitkv_check(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                        int64_t N, int64_t d, int causal, float softmax_scale, int64_t n_splits) {
    if (!q || !k || !v || !o) return FA_ERR_NULL_POINTER;
    fa_status st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if ((st = check_scale(softmax_scale)) != FA_OK) return st;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARGUMENT;
    if (n_splits < 1 || n_splits > kMaxParts) return FA_ERR_INVALID_ARGUMENT;
    if (o == q || o == k || o == v) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || (lse && !aligned(lse, 4)))
        return FA_ERR_MISALIGNED;
    return FA_OK;
}

struct SplitLayout {
    size_t off_lse, total;     // partial O at 0 (fp32 [n_splits, BH, N, d]), lse at off_lse
};

SplitLayout splitkv_layout(int64_t B, int64_t H, int64_t N, int64_t d, int64_t n_splits) {
    const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(H) * static_cast<size_t>(N);
    const size_t off_lse = round_up(static_cast<size_t>(n_splits) * rows * static_cast<size_t>(d) * 4, 256);
    return {off_lse, off_lse + round_up(static_cast<size_t>(n_splits) * rows * 4, 256)};
}

hipError_t splitkv_launch(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                          int64_t N, int64_t d, int causal, float softmax_scale, int64_t n_splits, uint8_t* base,
                          hipStream_t s) {
    const int BH = static_cast<int>(B * H), n = static_cast<int>(N), dd = static_cast<int>(d);
    const int n_tiles = (n + fa::kKeyTile - 1) / fa::kKeyTile;
    const int tps = (n_tiles + static_cast<int>(n_splits) - 1) / static_cast<int>(n_splits);
    const SplitLayout lay = splitkv_layout(B, H, N, d, n_splits);
    float* o32 = reinterpret_cast<float*>(base);
    float* lse_part = reinterpret_cast<float*>(base + lay.off_lse);
    // every (split, row) entry of o32 and lse_part is written by the partial
    // kernel (rows that see no key of a split get O = 0, lse = -inf) before the
    // merge reads it, so the buffer needs no clearing
    fa::FwdArgs a{fa::Kind::BF16, q, k, v, nullptr, nullptr, nullptr, nullptr, nullptr,
                  BH, n, padded_keys(n), dd, causal == 1, softmax_scale};
    a.o32 = o32;
    a.lse_part = lse_part;
    a.kt_lo = 0;
    a.kt_hi = n_tiles;
    a.tps = tps;
    a.n_splits = static_cast<int>(n_splits);
    hipError_t e = fa::launch_fwd(a, s);
    if (e == hipSuccess) e = fa::launch_merge(o32, lse_part, static_cast<int>(n_splits), o, lse, BH, n, dd, s);
    return e;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
    switch (s) {
        case FA_OK: return "ok";
        case FA_ERR_NULL_POINTER: return "a required pointer is NULL";
        case FA_ERR_INVALID_SHAPE: return "B, H, N must be >= 1 and B*H*ceil(N/64)*64*d < 2^31";
        case FA_ERR_UNSUPPORTED_HEAD_DIM: return "head dim must be 32, 64 or 128";
        case FA_ERR_INVALID_SCALE: return "softmax_scale must be finite and > 0";
        case FA_ERR_INVALID_DTYPE: return "unknown or unsupported dtype";
        case FA_ERR_MISALIGNED: return "tensor pointers must be 16-byte aligned (lse/scales 4-byte)";
        case FA_ERR_INVALID_ARGUMENT: return "invalid argument (causal must be 0 or 1; outputs must not alias inputs)";
        case FA_ERR_UNSUPPORTED_ARCH: return "current device is not gfx950 (MI355X)";
        case FA_ERR_OUT_OF_MEMORY: return "device workspace allocation failed";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_HIP: return "HIP runtime call failed";
        case FA_ERR_SCRATCH_LIMIT:
            return "the partial results need more than the library's static scratch buffer "
                   "(FA_NOALLOC_SCRATCH_BYTES); use fewer splits or the allocating entry point";
    }
    return "unknown status";
}

int fa_abi_version(void) { return FA_ABI_VERSION; }

fa_status fa_quant_fp8_e4m3(const void* x_bf16, uint8_t* x8, float* scale, int64_t BH, int64_t N, int64_t d,
                            void* stream) {
    if (!x_bf16 || !x8 || !scale) return FA_ERR_NULL_POINTER;
    fa_status st = check_shape(1, BH, N, d);
    if (st != FA_OK) return st;
    if (!aligned(x_bf16, 16) || !aligned(x8, 16) || !aligned(scale, 4)) return FA_ERR_MISALIGNED;
    if ((st = check_device()) != FA_OK) return st;
    return launch_status(fa::launch_quant_fp8(x_bf16, x8, scale, static_cast<int>(BH), static_cast<int>(N),
                                              static_cast<int>(d), static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                     const void* v_bf16, void* o_bf16, float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
                     int causal, float softmax_scale, void* stream) {
    if (!q8 || !q_scale || !k8 || !k_scale || !v_bf16 || !o_bf16) return FA_ERR_NULL_POINTER;
    fa_status st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if ((st = check_scale(softmax_scale)) != FA_OK) return st;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARGUMENT;
    if (o_bf16 == q8 || o_bf16 == k8 || o_bf16 == v_bf16) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v_bf16, 16) || !aligned(o_bf16, 16) ||
        !aligned(q_scale, 4) || !aligned(k_scale, 4) || (lse && !aligned(lse, 4)))
        return FA_ERR_MISALIGNED;
    if ((st = check_device()) != FA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int BH = static_cast<int>(B * H), n = static_cast<int>(N), dd = static_cast<int>(d);
    fa::FwdArgs a{fa::Kind::FP8, q8, k8, v_bf16, nullptr, o_bf16, lse, q_scale, k_scale,
                  BH, n, padded_keys(n), dd, causal == 1, softmax_scale};
    return launch_status(fa::launch_fwd(a, s));
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
                 int64_t d, int causal, float softmax_scale, fa_dtype dtype, void* stream) {
    if (!q || !k || !v || !o) return FA_ERR_NULL_POINTER;
    fa_status st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if ((st = check_scale(softmax_scale)) != FA_OK) return st;
    if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_FP8_E4M3 && dtype != FA_FP8_E4M3_PV)
        return FA_ERR_INVALID_DTYPE;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARGUMENT;
    if (o == q || o == k || o == v) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || (lse && !aligned(lse, 4)))
        return FA_ERR_MISALIGNED;
    if ((st = check_device()) != FA_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int BH = static_cast<int>(B * H), n = static_cast<int>(N), dd = static_cast<int>(d);
    if (dtype == FA_F32) {
        fa::FwdArgs a{fa::Kind::F32, q, k, v, nullptr, o, lse, nullptr, nullptr, BH, n, n, dd, causal == 1,
                      softmax_scale};
        return launch_status(fa::launch_fwd(a, s));
    }

    if (dtype == FA_FP8_E4M3_PV) {
        // e4m3 Q and K (per-tile fp32 scales), e4m3 V^T (power-of-two block exponents)
        const size_t codes = static_cast<size_t>(BH) * n * dd;
        const size_t n_scales = static_cast<size_t>(BH) * ((n + 63) / 64);
        const size_t v8b = static_cast<size_t>(BH) * dd * padded_keys(n);
        const size_t off_v8 = 0;
        const size_t off_vs = off_v8 + round_up(v8b, 256);
        const size_t off_q8 = off_vs + round_up(n_scales * dd, 256);
        const size_t off_k8 = off_q8 + round_up(codes, 256);
        const size_t off_qs = off_k8 + round_up(codes, 256);
        const size_t off_ks = off_qs + round_up(n_scales * 4, 256);
        const size_t total = off_ks + round_up(n_scales * 4, 256);
        void* ws = nullptr;
        if ((st = ws_alloc(&ws, total, s)) != FA_OK) return st;
        uint8_t* base = static_cast<uint8_t*>(ws);
        uint8_t* v8 = base + off_v8;
        uint8_t* vs = base + off_vs;
        uint8_t* q8 = base + off_q8;
        uint8_t* k8 = base + off_k8;
        float* qs = reinterpret_cast<float*>(base + off_qs);
        float* ks = reinterpret_cast<float*>(base + off_ks);
        hipError_t e = fa::launch_quant_v_pow2(v, v8, vs, BH, n, dd, s);
        if (e == hipSuccess) e = fa::launch_quant_fp8(q, q8, qs, BH, n, dd, s);
        if (e == hipSuccess) e = fa::launch_quant_fp8(k, k8, ks, BH, n, dd, s);
        if (e == hipSuccess) {
            fa::FwdArgs a{fa::Kind::FP8PV, q8, k8, v, v8, o, lse, qs, ks, BH, n, padded_keys(n), dd, causal == 1,
                          softmax_scale};
            a.v_scale = vs;
            e = fa::launch_fwd(a, s);
        }
        const hipError_t ef = ws_free(ws, s);
        if (e != hipSuccess) return launch_status(e);
        return ef == hipSuccess ? FA_OK : FA_ERR_HIP;
    }

    if (dtype == FA_BF16) {
        // one kernel, no workspace: V is read as it is
        fa::FwdArgs a{fa::Kind::BF16, q, k, v, nullptr, o, lse, nullptr, nullptr, BH, n, padded_keys(n), dd,
                      causal == 1, softmax_scale};
        return launch_status(fa::launch_fwd(a, s));
    }

    // FP8: one stream-ordered workspace for the e4m3 codes of Q and K and their per-tile scales
    const size_t codes = static_cast<size_t>(BH) * n * dd;
    const size_t n_scales = static_cast<size_t>(BH) * ((n + 63) / 64);
    const size_t off_q8 = 0;
    const size_t off_k8 = off_q8 + round_up(codes, 256);
    const size_t off_qs = off_k8 + round_up(codes, 256);
    const size_t off_ks = off_qs + round_up(n_scales * 4, 256);
    const size_t total = off_ks + round_up(n_scales * 4, 256);
    void* ws = nullptr;
    if ((st = ws_alloc(&ws, total, s)) != FA_OK) return st;
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint8_t* q8 = base + off_q8;
    uint8_t* k8 = base + off_k8;
    float* qs = reinterpret_cast<float*>(base + off_qs);
    float* ks = reinterpret_cast<float*>(base + off_ks);
    hipError_t e = fa::launch_quant_fp8(q, q8, qs, BH, n, dd, s);
    if (e == hipSuccess) e = fa::launch_quant_fp8(k, k8, ks, BH, n, dd, s);
    if (e == hipSuccess) {
        fa::FwdArgs a{fa::Kind::FP8, q8, k8, v, nullptr, o, lse, qs, ks, BH, n, padded_keys(n), dd, causal == 1,
                      softmax_scale};
        e = fa::launch_fwd(a, s);
    }
    const hipError_t ef = ws_free(ws, s);
    if (e != hipSuccess) return launch_status(e);
    return ef == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                         int64_t B, int64_t H, int64_t N, int64_t d, int64_t kv_begin, int64_t kv_end,
                         int causal, float softmax_scale, void* stream) {
    if (!q || !k || !v || !o_part || !lse_part) return FA_ERR_NULL_POINTER;
    fa_status st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if ((st = check_scale(softmax_scale)) != FA_OK) return st;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARGUMENT;
    if (kv_begin < 0 || kv_begin > kv_end || kv_end > N || kv_begin % fa::kKeyTile != 0 ||
        (kv_end % fa::kKeyTile != 0 && kv_end != N))
        return FA_ERR_INVALID_ARGUMENT;
    const void* outs[] = {o_part, lse_part};
    for (const void* x : outs)
        if (x == q || x == k || x == v) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_part, 16) || !aligned(lse_part, 4))
        return FA_ERR_MISALIGNED;
    if ((st = check_device()) != FA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int BH = static_cast<int>(B * H), n = static_cast<int>(N), dd = static_cast<int>(d);
    fa::FwdArgs a{fa::Kind::BF16, q, k, v, nullptr, nullptr, nullptr, nullptr, nullptr,
                  BH, n, padded_keys(n), dd, causal == 1, softmax_scale};
    a.o32 = o_part;
    a.lse_part = lse_part;
    a.kt_lo = static_cast<int>(kv_begin / fa::kKeyTile);
    a.kt_hi = static_cast<int>((kv_end + fa::kKeyTile - 1) / fa::kKeyTile);
    a.tps = a.kt_hi > a.kt_lo ? a.kt_hi - a.kt_lo : 1;
    a.n_splits = 1;
    return launch_status(fa::launch_fwd(a, s));
}

fa_status fa_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, void* o, float* lse,
                   int64_t B, int64_t H, int64_t N, int64_t d, void* stream) {
    if (!o_parts || !lse_parts || !o) return FA_ERR_NULL_POINTER;
    fa_status st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if (n_parts < 1 || n_parts > kMaxParts) return FA_ERR_INVALID_ARGUMENT;
    if (o == o_parts || o == lse_parts || lse == o_parts || lse == lse_parts) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned(o_parts, 16) || !aligned(o, 16) || !aligned(lse_parts, 4) || (lse && !aligned(lse, 4)))
        return FA_ERR_MISALIGNED;
    if ((st = check_device()) != FA_OK) return st;
    return launch_status(fa::launch_merge(o_parts, lse_parts, static_cast<int>(n_parts), o, lse,
                                          static_cast<int>(B * H), static_cast<int>(N), static_cast<int>(d),
                                          static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t N, int64_t d, int causal, float softmax_scale,
                         int64_t n_splits, void* stream) {
    fa_status st = splitkv_check(q, k, v, o, lse, B, H, N, d, causal, softmax_scale, n_splits);
    if (st != FA_OK) return st;
    if ((st = check_device()) != FA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if ((st = ws_alloc(&ws, splitkv_layout(B, H, N, d, n_splits).total, s)) != FA_OK) return st;
    const hipError_t e = splitkv_launch(q, k, v, o, lse, B, H, N, d, causal, softmax_scale, n_splits,
                                        static_cast<uint8_t*>(ws), s);
    const hipError_t ef = ws_free(ws, s);
    if (e != hipSuccess) return launch_status(e);
    return ef == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int64_t B, int64_t H, int64_t N, int64_t d, int causal, float softmax_scale,
                                 int64_t n_splits, void* stream) {
    fa_status st = splitkv_check(q, k, v, o, lse, B, H, N, d, causal, softmax_scale, n_splits);
    if (st != FA_OK) return st;
    if (splitkv_layout(B, H, N, d, n_splits).total > static_cast<size_t>(FA_NOALLOC_SCRATCH_BYTES))
        return FA_ERR_SCRATCH_LIMIT;
    if ((st = check_device()) != FA_OK) return st;
    void* base = nullptr;
    if (fa::scratch_address(&base) != hipSuccess) return FA_ERR_HIP;
    return launch_status(splitkv_launch(q, k, v, o, lse, B, H, N, d, causal, softmax_scale, n_splits,
                                        static_cast<uint8_t*>(base), static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t N, int64_t d, const uint8_t* block_mask,
                             int64_t mask_bh_stride, int causal, float softmax_scale, void* stream) {
    if (!q || !k || !v || !o || !block_mask) return FA_ERR_NULL_POINTER;
    fa_status st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if ((st = check_scale(softmax_scale)) != FA_OK) return st;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARGUMENT;
    const int64_t nb = (N + fa::kKeyTile - 1) / fa::kKeyTile;
    if (mask_bh_stride != 0 && mask_bh_stride != nb * nb) return FA_ERR_INVALID_ARGUMENT;
    if (o == q || o == k || o == v || o == block_mask) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || (lse && !aligned(lse, 4)))
        return FA_ERR_MISALIGNED;
    if ((st = check_device()) != FA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int BH = static_cast<int>(B * H), n = static_cast<int>(N), dd = static_cast<int>(d);
    const size_t n_lists = static_cast<size_t>(BH) * ((n + fa::kQueryTile - 1) / fa::kQueryTile);
    const size_t off_list = 0;
    const size_t off_cnt = off_list + round_up(n_lists * static_cast<size_t>(nb) * 4, 256);
    const size_t total = off_cnt + round_up(n_lists * 4, 256);
    void* ws = nullptr;
    if ((st = ws_alloc(&ws, total, s)) != FA_OK) return st;
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint32_t* list = reinterpret_cast<uint32_t*>(base + off_list);
    int* cnt = reinterpret_cast<int*>(base + off_cnt);
    hipError_t e = fa::launch_bs_plan(block_mask, mask_bh_stride, BH, n, causal == 1, list, cnt, s);
    if (e == hipSuccess) {
        fa::FwdArgs a{fa::Kind::BF16, q, k, v, nullptr, o, lse, nullptr, nullptr,
                      BH, n, padded_keys(n), dd, causal == 1, softmax_scale};
        a.bs_list = list;
        a.bs_count = cnt;
        a.bs_stride = static_cast<int>(nb);
        e = fa::launch_fwd(a, s);
    }
    const hipError_t ef = ws_free(ws, s);
    if (e != hipSuccess) return launch_status(e);
    return ef == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_quant_v_pow2(const void* v_bf16, uint8_t* v8, uint8_t* v_scale, int64_t BH, int64_t N, int64_t d,
                          void* stream) {
    if (!v_bf16 || !v8 || !v_scale) return FA_ERR_NULL_POINTER;
    fa_status st = check_shape(1, BH, N, d);
    if (st != FA_OK) return st;
    if (!aligned(v_bf16, 16) || !aligned(v8, 16)) return FA_ERR_MISALIGNED;
    if ((st = check_device()) != FA_OK) return st;
    return launch_status(fa::launch_quant_v_pow2(v_bf16, v8, v_scale, static_cast<int>(BH), static_cast<int>(N),
                                                 static_cast<int>(d), static_cast<hipStream_t>(stream)));
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                 int causal, float softmax_scale, fa_dtype dtype, void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL_POINTER;
    fa_status st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if ((st = check_scale(softmax_scale)) != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_INVALID_DTYPE;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARGUMENT;
    const void* ins[] = {q, k, v, o, dout, lse};
    const void* outs[] = {dq, dk, dv};
    for (const void* x : outs) {
        for (const void* y : ins)
            if (x == y) return FA_ERR_INVALID_ARGUMENT;
    }
    if (dq == dk || dq == dv || dk == dv) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
        return FA_ERR_MISALIGNED;
    if ((st = check_device()) != FA_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int BH = static_cast<int>(B * H), n = static_cast<int>(N), dd = static_cast<int>(d);
    // d = 128 reads Q^T, dO^T and K^T out of natural rows (transposing LDS reads);
    // d = 32 and 64 take transposed copies
    const bool copies = dd != 128;
    const size_t tb = copies ? round_up(vt_bytes(BH, n, dd), 256) : 0;
    const size_t vec = round_up(static_cast<size_t>(BH) * n * 4, 256);
    void* ws = nullptr;
    if ((st = ws_alloc(&ws, 3 * tb + 2 * vec, s)) != FA_OK) return st;
    uint8_t* base = static_cast<uint8_t*>(ws);
    void* qt = copies ? base : nullptr;
    void* dot = copies ? base + tb : nullptr;
    void* kt = copies ? base + 2 * tb : nullptr;
    float* lse2 = reinterpret_cast<float*>(base + 3 * tb);
    float* dsum = reinterpret_cast<float*>(base + 3 * tb + vec);
    hipError_t e = hipSuccess;
    if (copies) {
        e = fa::launch_transpose_v(q, qt, BH, n, dd, s);
        if (e == hipSuccess) e = fa::launch_transpose_v(dout, dot, BH, n, dd, s);
        if (e == hipSuccess) e = fa::launch_transpose_v(k, kt, BH, n, dd, s);
    }
    if (e == hipSuccess) {
        fa::BwdArgs a{q, k, v, o, dout, lse, qt, dot, kt, lse2, dsum, dq, dk, dv,
                      BH, n, padded_keys(n), dd, causal == 1, softmax_scale};
        e = fa::launch_bwd(a, s);
    }
    const hipError_t ef = ws_free(ws, s);
    if (e != hipSuccess) return launch_status(e);
    return ef == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
