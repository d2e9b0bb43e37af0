// Internal interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum class Kind { F32, BF16, FP8, FP8PV };

struct FwdArgs {
    Kind kind;
    const void* q;          // f32 / bf16 / e4m3 codes
    const void* k;
    const void* v;          // f32 or bf16
    const void* vt;         // FP8PV only: e4m3 V^T from launch_quant_v_pow2, [BH, d, np] bytes
    void* o;                // f32 or bf16
    float* lse;             // may be null
    const float* q_scale;   // FP8 only: [BH, ceil(N/64)]
    const float* k_scale;
    int BH;
    int N;
    int np;                 // row length of vt (FP8PV): N rounded up to the 64-key tile
    int d;
    bool causal;
    float softmax_scale;
    // Partial results (bf16 only): when o32 is set, the kernel computes, for
    // each split s < n_splits, attention over key tiles
    // [kt_lo + s*tps, min(kt_hi, kt_lo + (s+1)*tps)) and writes O normalised over
    // those keys to o32 [n_splits, BH, N, d] (fp32) and its lse to lse_part
    // [n_splits, BH, N] (-inf where no key is visible); o and lse are not written.
    float* o32 = nullptr;
    float* lse_part = nullptr;
    int kt_lo = 0, kt_hi = 0, tps = 0, n_splits = 0;
    // Block-sparse (bf16 only): when bs_list is set, each (bh, 256-query tile)
    // visits only the key tiles listed by launch_bs_plan.
    const uint32_t* bs_list = nullptr;
    const int* bs_count = nullptr;
    int bs_stride = 0;
    // FP8PV: block-exponent bytes of the e4m3 V^T, [BH, ceil(N/64), d]
    const uint8_t* v_scale = nullptr;
};

// Query rows per workgroup of the bf16/FP8 attention kernel (four 64-row blocks).
constexpr int kQueryTile = 256;

// Enqueue the planning pass of the block-sparse kernel: for every (bh, 256-query
// tile) the key tiles any of its four 64-query blocks may see under the 0/1
// table mask[bh * mask_bh_stride + qb * nb + kb] (nb = ceil(N/64); causal drops
// kb > qb).  list holds BH * ceil(N/256) * nb entries, count BH * ceil(N/256).
hipError_t launch_bs_plan(const uint8_t* mask, long long mask_bh_stride, int BH, int N, bool causal,
                          uint32_t* list, int* count, hipStream_t stream);

// Enqueue the forward kernel on `stream`; returns the launch status.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// Keys per tile of the bf16/FP8 attention kernel; V^T rows are padded to a multiple of it.
constexpr int kKeyTile = 64;

// Enqueue the merge of n_parts partial results (o_parts [n_parts, BH, N, d]
// fp32, lse_parts [n_parts, BH, N]) into bf16 o [BH, N, d] and lse (may be null):
// lse = ln sum_g exp(lse_g), O = sum_g exp(lse_g - lse) O_g.
hipError_t launch_merge(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse,
                        int BH, int N, int d, hipStream_t stream);

// Enqueue the transposition of a bf16 [BH, N, d] tensor into [BH, d, np] (np = N
// rounded up to kKeyTile, padding zero), keys permuted within each tile into the
// order the backward kernels' LDS layouts use.  The output must hold BH * d * np
// bf16 values.
hipError_t launch_transpose_v(const void* v, void* vt, int BH, int N, int d, hipStream_t stream);

struct BwdArgs {
    const void* q;          // bf16 [BH, N, d]
    const void* k;
    const void* v;
    const void* o;          // forward output
    const void* dout;       // upstream gradient
    const float* lse;       // forward logsumexp [BH, N]
    const void* qt;         // Q^T, dO^T, K^T from launch_transpose_v, [BH, d, np] each
    const void* dot;
    const void* kt;
    float* lse2;            // workspace [BH, N]: lse * log2(e)
    float* dsum;            // workspace [BH, N]: rowsum(dO * O)
    void* dq;               // bf16 [BH, N, d]
    void* dk;
    void* dv;
    int BH;
    int N;
    int np;
    int d;
    bool causal;
    float softmax_scale;
};

// Enqueue the backward kernels (row statistics, dK/dV, dQ) on `stream`.
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

// Enqueue the power-of-two e4m3 quantisation of a bf16 V [BH, N, d] for the
// FP8 P*V kernel: v8 [BH, d, np] bytes (np = N rounded up to 64, keys of each
// tile in the order the kernel's P operand uses), vscale [BH, ceil(N/64), d]
// bytes 127 - e with e the largest integer (clipped to +-127) for which the
// tile column's amax * 2^e <= 448.
hipError_t launch_quant_v_pow2(const void* v, uint8_t* v8, uint8_t* vscale, int BH, int N, int d,
                              hipStream_t stream);

// Enqueue the per-64-row-tile e4m3fn quantisation of a bf16 [BH, N, d] tensor.
hipError_t launch_quant_fp8(const void* x_bf16, uint8_t* x8, float* scale,
                            int BH, int N, int d, hipStream_t stream);

}  // namespace fa
