// Attention backward for gfx950 (MI355X): dQ, dK, dV of
// O = softmax(scale * Q K^T [causally masked]) V for an upstream gradient dO.
//
// The forward pass keeps no probabilities; the backward pass recomputes them
// from Q, K and the per-row logsumexp the forward wrote (the Triton
// walkthrough page, section 2.2: intermediate results are recomputed in the
// backward pass instead of stored).  With P = exp(scale * S - lse):
//
//   dV = P^T dO,   dP = dO V^T,   D_i = sum_k dO_ik O_ik,
//   dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
//
// Work is split so that no two workgroups write the same output row (the tag
// page, excerpt on V2: the work of the backward pass is reassigned to cut
// synchronisation between thread blocks):
//
//  * bwd_prep_kernel: D_i and lse_i * log2(e) per query row.
//  * At d = 128 two kernels on the forward's ping-pong schedule replace the
//    three below (bwd_dq_pp_kernel for dQ; bwd_kvf_kernel for dK and dV
//    together, S computed once): two wave groups one slot apart, so that one
//    wave of each SIMD issues matrix-core work while the other runs the exp
//    and dS arithmetic.
//  * bwd_dq_kernel: query-stationary, the forward's layout.  A workgroup
//    holds 256 queries (32 per wave, Q and dO in registers as MFMA B
//    operands) and streams 64-key tiles of K, V and K^T through LDS;
//    S^T = K Q^T and dP^T = V dO^T give every lane the scores of one query,
//    so lse and D are one value per lane, and dS^T lands in the B-operand
//    layout of dQ^T += K^T dS^T.
//  * bwd_kv_kernel<.., 0> (dV) and <.., 1> (dK): key-stationary.  A
//    workgroup holds 256 keys (32 per wave, K and V in registers) and streams
//    64-query tiles of Q, dO^T (dV) or Q, dO, Q^T, lse and D (dK) through
//    LDS; S = Q K^T and dP = dO V^T give every lane the scores of one key,
//    and P and dS land in the B-operand layout of dV^T += dO^T P and
//    dK^T += Q^T dS.  Splitting the two keeps each under 256 VGPRs, two
//    waves per SIMD, at the price of computing S twice.
//
// The transposed operands (K^T, Q^T, dO^T) come from the same pre-pass the
// forward uses for V^T, with rows permuted within each 16-group so that a
// 16-byte LDS read feeds one MFMA A operand.  P and dS are rounded to bf16
// for the MFMAs; everything else accumulates in fp32.  Causal: tiles that
// lie entirely above the diagonal are skipped, and only tiles that cross it
// (or the sequence end) compare indices.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

struct BParams {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    const uint8_t* dout;
    const uint8_t* qt;       // Q^T  [BH, D, np], rows permuted within each 16-group
    const uint8_t* dot;      // dO^T [BH, D, np]
    const uint8_t* kt;       // K^T  [BH, D, np]
    const float* lse2;       // lse * log2(e)   [BH, N]
    const float* dsum;       // D = rowsum(dO * O) [BH, N]
    uint8_t* dq;
    uint8_t* dk;
    uint8_t* dv;
    int BH;
    int N;
    int np;
    int n_tiles;             // workgroups per (b, h)
    float c_log2;            // softmax_scale * log2(e)
    float scale;
};

// Natural-layout row tiles read with the transposing LDS read (d = 128): a
// tile of R rows of 256 bytes, row r's 16-byte granule g at granule
// tr_granule(r, g), an XOR and so its own inverse.  The transposing reads
// take, per 32 lanes, four consecutive rows x 64 bytes; the swizzle puts
// those four pieces on four distinct quarters of the 64 LDS banks.
__device__ __forceinline__ int tr_granule(int row, int g) { return g ^ (4 * (row & 3)); }

// Per-lane LDS-DMA source offset of the first of a wave's copy blocks of such
// a tile: block (w & 3) + 4i holds rows 4 ((w & 3) + 4i) .. +3, so the blocks
// of one wave are 16 rows (4 KiB of source) apart.
__device__ __forceinline__ uint32_t tr_copy_offset(int w, int lane) {
    const int row = 4 * (w & 3) + (lane >> 4);
    return static_cast<uint32_t>(row * 256 + 16 * tr_granule(row, lane & 15));
}

// LDS byte offset, within such a tile, of the first transposing read of the
// A operand X^T (32 head dims 32 db .. + 31, 16 rows of chunk 0) of
// acc^T += X^T Y: lane 16g + 4r + j reads dims 32 db + 16 (g & 1) + 4j .. +3
// of row 4 (g >> 1) + r; the second read of a chunk is 8 rows further on and
// chunk cc is 16 cc rows further.  The eight rows a lane then holds are the
// ones the MFMA's k-slots 8h .. 8h+7 meet in a score-layout Y fragment.
__device__ __forceinline__ uint32_t tr_read_offset(int lane, int db) {
    const int g = lane >> 4, r = (lane >> 2) & 3, j = lane & 3;
    return (4 * (g >> 1) + r) * 256 + 64 * (db ^ r) + 16 * (2 * (g & 1) + (j >> 1)) + 8 * (j & 1);
}

// Row tiles read both ways (rows of 256 bytes, d = 128): by 16-byte row reads
// (the A operand of an MFMA over the row dimension: lane l reads row l % 32,
// granule 2i + l / 32) and by the transposing read above.  Granule g of row r
// sits at xr_granule(r, g) = g ^ (4 (r & 3) + ((r >> 2) & 3)): four
// consecutive rows fall on four bank quarters, as the transposing reads need,
// and eight consecutive rows on eight distinct granules, as the row reads
// need.  (Measured per CU: 4.4 cycles per 1 KiB row read against 4.1 on
// padded rows and 14.1 under tr_granule; 3.9 cycles per transposing read, as
// under tr_granule.)
__device__ __forceinline__ int xr_granule(int row, int g) { return g ^ (4 * (row & 3) + ((row >> 2) & 3)); }
__device__ __forceinline__ uint32_t xr_copy_offset(int w, int lane) {
    const int row = 4 * (w & 3) + (lane >> 4);
    return static_cast<uint32_t>(row * 256 + 16 * xr_granule(row, lane & 15));
}
// The transposing reads of such a tile (tr_read_offset's pattern): the offset of
// the first read; the second read of a chunk (8 rows further on) is at
// xr_read_offset + xr_hi_delta, because for these rows xr_granule differs from
// the first read's by 2 in the granule index.
__device__ __forceinline__ uint32_t xr_read_offset(int lane, int db) {
    const int g = lane >> 4, r = (lane >> 2) & 3, j = lane & 3;
    const int row = 4 * (g >> 1) + r;
    return row * 256 + 16 * xr_granule(row, 4 * db + 2 * (g & 1) + (j >> 1)) + 8 * (j & 1);
}
__device__ __forceinline__ int xr_hi_delta(int lane) { return 8 * 256 + (((lane >> 4) & 1) ? -32 : 32); }

// ===========================================================================
// Pre-pass: D_i = sum_k dO_ik O_ik and lse_i * log2(e), one row per group of
// D/8 lanes (16 bytes of O and dO per lane).
// ===========================================================================
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint8_t* __restrict__ o, const uint8_t* __restrict__ dout,
                                                       const float* __restrict__ lse, float* __restrict__ lse2,
                                                       float* __restrict__ dsum, long long rows) {
    constexpr int LPR = D / 8;                           // lanes per row
    const long long row = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.0f;
    if (row < rows) {
        const size_t off = (static_cast<size_t>(row) * D + 8 * part) * 2;
        const u32x4 a = ld16(o + off), b = ld16(dout + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), acc);
            acc = fmaf(__uint_as_float(a[e] & 0xFFFF0000u), __uint_as_float(b[e] & 0xFFFF0000u), acc);
        }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (row < rows && part == 0) {
        dsum[row] = acc;
        lse2[row] = lse[row] * kLog2e;
    }
}

// ===========================================================================
// dQ: 8 waves x 32 queries, 64-key tiles of K, V and K^T in a 2-stage LDS ring.
// ===========================================================================
template <int D>
struct DqCfg {
    static constexpr int NW = 8;
    static constexpr int NT = 64 * NW;
    static constexpr int BM = 32 * NW;
    static constexpr int BN = kKeyTile;
    static constexpr int KROW = 2 * D + 16;              // bytes per K / V row in LDS (padded)
    static constexpr int TROW = 2 * BN + 16;             // bytes per K^T row in LDS (padded)
    static constexpr int KBYTES = dma_region_bytes(BN * KROW);
    static constexpr int TBYTES = dma_region_bytes(D * TROW);
    static constexpr int STAGE = 2 * KBYTES + TBYTES;
    static constexpr int QREGS = D / 16;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BParams p) {
    using C = DqCfg<D>;
    constexpr int BM = C::BM, BN = C::BN, NT = C::NT;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int N = p.N;
    int qt = blockIdx.x / p.BH;
    const int bh = blockIdx.x - qt * p.BH;
    if (CAUSAL) qt = p.n_tiles - 1 - qt;                 // heaviest query tiles first
    const int q0 = qt * BM, qw0 = q0 + 32 * w, my_q = qw0 + l32;

    const size_t slice = static_cast<size_t>(bh) * N * D;
    const uint8_t* kg = p.k + slice * 2;
    const uint8_t* vg = p.v + slice * 2;
    const uint8_t* ktg = p.kt + static_cast<size_t>(bh) * D * p.np * 2;

    // Q and dO rows of this lane's query: B operands (k-slots = d)
    u32x4 qf[C::QREGS], gf[C::QREGS];
    float lse2_q = 0.0f, d_q = 0.0f;
    {
        const bool ok = my_q < N;
        const size_t off = (slice + static_cast<size_t>(my_q) * D) * 2;
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i) {
            qf[i] = ok ? ld16(p.q + off + 2 * (16 * i + 8 * h)) : u32x4{0, 0, 0, 0};
            gf[i] = ok ? ld16(p.dout + off + 2 * (16 * i + 8 * h)) : u32x4{0, 0, 0, 0};
        }
        if (ok) {
            lse2_q = p.lse2[static_cast<size_t>(bh) * N + my_q];
            d_q = p.dsum[static_cast<size_t>(bh) * N + my_q];
        }
    }

    const int n_all = (N + BN - 1) / BN;
    const int n_kt = CAUSAL ? min(n_all, (min(q0 + BM, N) + BN - 1) / BN) : n_all;
    const int j_last = CAUSAL ? min(n_kt - 1, (qw0 + 31) / BN) : n_kt - 1;

    // Tiles go global -> LDS directly (buffer loads to LDS): a stage is K rows,
    // V rows (272-byte stride: 16 granules + one pad) and K^T rows (144 bytes:
    // 8 + 1), NB contiguous 1 KiB blocks, block b copied by wave b mod 8.  The
    // copy of tile j+1 is issued before tile j is computed and waited for
    // before the barrier that ends it; the hardware range check zero-fills
    // keys past the end of the sequence.
    static_assert(C::KROW == 2 * D + 16 && C::TROW == 144, "LDS-DMA layout");
    constexpr int NB_K = C::KBYTES / 1024, NB = 2 * NB_K + C::TBYTES / 1024, PER_W = (NB + 7) / 8;
    uint32_t doff[PER_W];
    int dn = 0;
#pragma unroll
    for (int i = 0; i < PER_W; ++i) {
        const int b = w + 8 * i;
        doff[i] = 0x40000000u;
        if (b < NB) {
            doff[i] = b < 2 * NB_K ? dma_lane_offset(b % NB_K, lane, D / 8, D * 2, BN)
                                   : dma_lane_offset(b - 2 * NB_K, lane, BN / 8, p.np * 2, D);
            dn = i + 1;
        }
    }
    const uint32_t smem_lds = lds_address(smem);
    auto copy_tile = [&](int t) {
        const int n0 = t * BN;
        const uint32_t valid = static_cast<uint32_t>(min(N - n0, BN)) * D * 2;
        const u32x4 kr = buffer_words(kg + static_cast<size_t>(n0) * D * 2, valid);
        const u32x4 vr = buffer_words(vg + static_cast<size_t>(n0) * D * 2, valid);
        const u32x4 tr = buffer_words(ktg + static_cast<size_t>(n0) * 2, (static_cast<uint32_t>(D) * p.np - n0) * 2);
        const uint32_t stage = smem_lds + (t & 1) * C::STAGE;
#pragma unroll
        for (int i = 0; i < PER_W; ++i) {
            const int b = w + 8 * i;
            if (i < dn) {
                poison_block(stage + 1024 * b);
                lds_dma16(stage + 1024 * b, b < NB_K ? kr : (b < 2 * NB_K ? vr : tr), doff[i]);
            }
        }
    };

    f32x16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

    // one 32-key block kb of tile j: S^T, dP^T, dS^T, then its share of dQ^T
    auto compute = [&](int j, int kb, bool masked) {
        const uint8_t* ks = smem + (j & 1) * C::STAGE;
        const uint8_t* vs = ks + C::KBYTES;
        const uint8_t* ts = vs + C::KBYTES;
        const int n0 = j * BN;
        f32x16 s = {}, dp = {};
        const uint8_t* kr = ks + (32 * kb + l32) * C::KROW + 16 * h;
        const uint8_t* vr = vs + (32 * kb + l32) * C::KROW + 16 * h;
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ld16(kr + 32 * i)),
                                                       __builtin_bit_cast(bf16x8, qf[i]), s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ld16(vr + 32 * i)),
                                                        __builtin_bit_cast(bf16x8, gf[i]), dp, 0, 0, 0);
        }
        float ds[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float pr = fast_exp2(fmaf(s[v], p.c_log2, -lse2_q));
            if (masked) {
                const int key = n0 + 32 * kb + acc_row(v, h);
                if (key >= N || (CAUSAL && key > my_q)) pr = 0.0f;
            }
            ds[v] = pr * (dp[v] - d_q);
        }
        bf16x8 dsf[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int t = 0; t < 8; ++t) dsf[cc][t] = static_cast<__bf16>(ds[8 * cc + t]);
        const uint8_t* tr = ts + l32 * C::TROW + 16 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, ld16(tr + 32 * db * C::TROW + 32 * (2 * kb + cc))), dsf[cc], dq[db], 0,
                    0, 0);
    };
    auto compute_block = [&](int j, int kb) {
        if (j > j_last) return;
        // only the last tile of this wave can cross the diagonal or the sequence end
        const int n0 = j * BN;
        compute(j, kb, j == j_last && ((CAUSAL && n0 + BN - 1 > qw0) || n0 + BN > N));
    };

    copy_tile(0);
    wait_lds_dma();
    __syncthreads();
    for (int j = 0; j < n_kt; ++j) {
        const bool more = j + 1 < n_kt;
        if (more) copy_tile(j + 1);
        compute_block(j, 0);
        compute_block(j, 1);
        if (more) wait_lds_dma();
        __syncthreads();
    }

    if (my_q < N) {
        uint8_t* orow = p.dq + (slice + static_cast<size_t>(my_q) * D) * 2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(dq[db][4 * g + e] * p.scale);
                *reinterpret_cast<bf16x4*>(orow + 2 * (32 * db + 8 * g + 4 * h)) = out;
            }
    }
}

// ===========================================================================
// dQ at d = 128 on the forward's ping-pong schedule.  Waves 0-3 (group A) and
// 4-7 (group B) sit one per SIMD each and run one slot apart, so that each
// SIMD holds one wave issuing matrix-core work while the other runs vector
// work.  Per wave, for 32-key tiles t:
//   M_t = { dQ^T += K_{t-1}^T dS_{t-1}^T,  S_t^T = K_t Q^T,  dP_t^T = V_t dO^T }
//   V_t = { P = exp2(S c - lse2), dS^T = P (dP - D), packed to bf16 }
// Group A runs op k in slot k, group B in slot k+1.  K and V rows of tile t
// are read in slots 2t and 2t+1; the K rows of tile t again, in a second copy
// read with the transposing LDS read (the K^T operand of dQ^T), in slots 2t+2
// and 2t+3.  Group B copies KV_{j+2} and KT_{j+1} in its vector slot 2j+2 into
// the stages the tiles two before left, and waits for them at the end of slot
// 2j+3, before the barrier after which group A reads them.
// ===========================================================================
constexpr int kDqSlotKeys = 64;                          // keys per slot of the d = 128 dQ kernel
template <int BN_>
struct DqPPCfg {
    static constexpr int D = 128, NW = 8, NT = 64 * NW, BM = 32 * NW, BN = BN_;
    static constexpr int KROW = 2 * D + 16;              // K / V row in LDS: 16 granules + 1 pad
    static constexpr int KREG = dma_region_bytes(BN * KROW);          // K, V: 9 KiB each (17 at BN = 64)
    static constexpr int KV_BLOCKS = (2 * KREG / 1024 + 3) / 4 * 4;   // whole groups of four copy blocks
    static constexpr int KT_BLOCKS = BN * 256 / 1024;                 // K rows, natural and swizzled
    static constexpr int KVSTAGE = KV_BLOCKS * 1024, KTSTAGE = KT_BLOCKS * 1024;
    static constexpr int SMEM = 2 * KVSTAGE + 2 * KTSTAGE;
    static constexpr int QREGS = D / 16;
    static constexpr int AHEAD = 6;
};

template <bool CAUSAL, int BN_>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_pp_kernel(BParams p) {
    using C = DqPPCfg<BN_>;
    constexpr int KB = BN_ / 32;                         // 32-key blocks per tile
    constexpr int D = C::D, BM = C::BM, BN = C::BN;
    static_assert(C::KT_BLOCKS % 4 == 0, "LDS-DMA layout");
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::SMEM];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, grp = w >> 2, h = lane >> 5, l32 = lane & 31;
    const int N = p.N;
    int qt = blockIdx.x / p.BH;
    const int bh = blockIdx.x - qt * p.BH;
    if (CAUSAL) qt = p.n_tiles - 1 - qt;                 // heaviest query tiles first
    const int q0 = qt * BM, qw0 = q0 + 32 * w, my_q = qw0 + l32;

    const size_t slice = static_cast<size_t>(bh) * N * D;
    const uint8_t* kg = p.k + slice * 2;
    const uint8_t* vg = p.v + slice * 2;

    // Q and dO rows of this lane's query (B operands), its lse2 and D
    u32x4 qf[C::QREGS], gf[C::QREGS];
    float lse2_q = 0.0f, d_q = 0.0f;
    {
        const bool ok = my_q < N;
        const size_t off = (slice + static_cast<size_t>(my_q) * D) * 2;
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i) {
            qf[i] = ok ? ld16(p.q + off + 2 * (16 * i + 8 * h)) : u32x4{0, 0, 0, 0};
            gf[i] = ok ? ld16(p.dout + off + 2 * (16 * i + 8 * h)) : u32x4{0, 0, 0, 0};
        }
        if (ok) {
            lse2_q = p.lse2[static_cast<size_t>(bh) * N + my_q];
            d_q = p.dsum[static_cast<size_t>(bh) * N + my_q];
        }
    }

    const int n_all = (N + BN - 1) / BN;
    const int n_kt = CAUSAL ? min(n_all, (min(q0 + BM, N) + BN - 1) / BN) : n_all;
    // last key tile with a key at or before this wave's last query
    const int j_last = CAUSAL ? min(n_kt - 1, (qw0 + 31) / BN) : n_kt - 1;
    uint32_t lane_to[D / 32];                       // transposing reads of the K^T operand
#pragma unroll
    for (int db = 0; db < D / 32; ++db) lane_to[db] = tr_read_offset(lane, db);

    // ---- tile copies (group B, wave w & 3 copies blocks (w & 3) + 4i)
    const uint32_t smem_lds = lds_address(smem);
    const uint32_t kvbase = smem_lds, ktbase = smem_lds + 2 * C::KVSTAGE;
    constexpr int KV_PER_W = C::KV_BLOCKS / 4, KT_PER_W = C::KT_BLOCKS / 4, KREG_BLOCKS = C::KREG / 1024;
    uint32_t kv_off[KV_PER_W], kt_off = 0;
    if (grp == 1) {
#pragma unroll
        for (int i = 0; i < KV_PER_W; ++i) {
            const int b = (w & 3) + 4 * i;            // K rows, then V rows, KREG_BLOCKS blocks each
            kv_off[i] = dma_lane_offset(b % KREG_BLOCKS, lane, D / 8, D * 2, b < 2 * KREG_BLOCKS ? BN : 0);
        }
        kt_off = tr_copy_offset(w, lane);
    }
    auto copy_kv = [&](int t) {                     // K_t, V_t rows into KV stage t % 2
        const int n0 = t * BN;
        const uint32_t valid = static_cast<uint32_t>(min(N - n0, BN)) * D * 2;
        const u32x4 kr = buffer_words(kg + static_cast<size_t>(n0) * D * 2, valid);
        const u32x4 vr = buffer_words(vg + static_cast<size_t>(n0) * D * 2, valid);
        const uint32_t st = kvbase + (t & 1) * C::KVSTAGE + 1024 * (w & 3);
#pragma unroll
        for (int i = 0; i < KV_PER_W; ++i) {
            poison_block(st + 4096 * i);
            lds_dma16(st + 4096 * i, (w & 3) + 4 * i < KREG_BLOCKS ? kr : vr, kv_off[i]);
        }
    };
    auto copy_kt = [&](int t) {                     // K_t rows, swizzled, into KT stage t % 2
        const int n0 = t * BN;
        const u32x4 r = buffer_words(kg + static_cast<size_t>(n0) * D * 2, static_cast<uint32_t>(min(N - n0, BN)) * D * 2);
        const uint32_t st = ktbase + (t & 1) * C::KTSTAGE + 1024 * (w & 3);
#pragma unroll
        for (int i = 0; i < KT_PER_W; ++i) {
            poison_block(st + 4096 * i);
            lds_dma16(st + 4096 * i, r, kt_off + 4096 * i);
        }
    };

    f32x16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};
    f32x16 s[KB], dp[KB];
    bf16x8 dsf[2 * KB];

    // S^T and dP^T of tile t (32-key blocks kb)
    auto op_s = [&](int t) {
        const uint8_t* kr = smem + (t & 1) * C::KVSTAGE + l32 * C::KROW + 16 * h;
        const uint8_t* vr = kr + C::KREG;
        bf16x8 a[2 * KB * C::QREGS];
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                a[2 * (KB * i + kb)] = __builtin_bit_cast(bf16x8, ld16(kr + 32 * kb * C::KROW + 32 * i));
                a[2 * (KB * i + kb) + 1] = __builtin_bit_cast(bf16x8, ld16(vr + 32 * kb * C::KROW + 32 * i));
            }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s[kb] = f32x16{};
            dp[kb] = f32x16{};
        }
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2 * (KB * i + kb)], __builtin_bit_cast(bf16x8, qf[i]),
                                                               s[kb], 0, 0, 0);
                dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2 * (KB * i + kb) + 1],
                                                                __builtin_bit_cast(bf16x8, gf[i]), dp[kb], 0, 0, 0);
            }
        pipeline_lds_mfma<2 * KB * C::QREGS, C::AHEAD>();
    };
    // dS^T of tile t (the key index of register v is t BN + acc_row(v, h))
    auto op_v = [&](int t, bool masked) {
        const int lim = min(N - 1, CAUSAL ? my_q : N - 1) - t * BN - 4 * h;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float ds[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float pr = fast_exp2(fmaf(s[kb][v], p.c_log2, -lse2_q));
                if (masked && 32 * kb + 8 * (v >> 2) + (v & 3) > lim) pr = 0.0f;
                ds[v] = pr * (dp[kb][v] - d_q);
            }
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int e = 0; e < 8; ++e) dsf[2 * kb + cc][e] = static_cast<__bf16>(ds[8 * cc + e]);
        }
    };
    // dQ^T += K_t^T dS_t^T
    auto op_dq = [&](int t) {
        const lds_u8* ts = (const lds_u8*)smem + 2 * C::KVSTAGE + (t & 1) * C::KTSTAGE;
        constexpr int NC = 2 * KB;                      // 16-key chunks of the tile
        bf16x8 a[NC * (D / 32)];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) {
                const i16x4 lo = ds_read_tr16(ts + lane_to[db] + 16 * cc * 256);
                const i16x4 hi = ds_read_tr16(ts + lane_to[db] + (16 * cc + 8) * 256);
                a[NC * db + cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int cc = 0; cc < NC; ++cc)
                dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[NC * db + cc], dsf[cc], dq[db], 0, 0, 0);
        pipeline_lds_mfma<NC * (D / 32), C::AHEAD, 2>();
    };
    auto masked_tile = [&](int t) { return (CAUSAL && t * BN + BN - 1 > qw0) || t * BN + BN > N; };
    auto slot_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: group B copies KV_0 and waits; everyone meets at barrier 0
    if (grp == 1) {
        copy_kv(0);
        wait_lds_dma();
    }
    lds_barrier();

    const bool last_masked = masked_tile(j_last);
    if (grp == 0) {
        // A: M_0 | V_0 M_1 | ... | V_{n-1} M_n | idle
        op_s(0);
        slot_end();
        for (int j = 0; j < j_last; ++j) {
            op_v(j, false);
            slot_end();
            op_dq(j);
            __builtin_amdgcn_sched_barrier(0);
            op_s(j + 1);
            slot_end();
        }
        op_v(j_last, last_masked);
        slot_end();
        op_dq(j_last);
        slot_end();
        for (int j = j_last + 1; j < n_kt; ++j) {     // past the diagonal: slots only
            slot_end();
            slot_end();
        }
        slot_end();
    } else {
        // B: copies | M_0 | V_0 + copies, M_1 | ... | V_{n-1} + copies, M_n
        if (1 < n_kt) copy_kv(1);
        copy_kt(0);
        slot_end();
        op_s(0);
        wait_lds_dma();
        slot_end();
        auto copies = [&](int j) {
            if (j + 2 < n_kt) copy_kv(j + 2);
            if (j + 1 < n_kt) copy_kt(j + 1);
        };
        for (int j = 0; j < j_last; ++j) {
            op_v(j, false);
            copies(j);
            slot_end();
            op_dq(j);
            __builtin_amdgcn_sched_barrier(0);
            op_s(j + 1);
            wait_lds_dma();
            slot_end();
        }
        op_v(j_last, last_masked);
        copies(j_last);
        slot_end();
        op_dq(j_last);
        wait_lds_dma();
        slot_end();
        for (int j = j_last + 1; j < n_kt; ++j) {     // past the diagonal: copies for the others
            copies(j);
            slot_end();
            wait_lds_dma();
            slot_end();
        }
    }

    if (my_q < N) {
        uint8_t* orow = p.dq + (slice + static_cast<size_t>(my_q) * D) * 2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(dq[db][4 * g + e] * p.scale);
                *reinterpret_cast<bf16x4*>(orow + 2 * (32 * db + 8 * g + 4 * h)) = out;
            }
    }
}

// ===========================================================================
// dV and dK as two key-stationary kernels of 8 waves x 32 keys (two waves per
// SIMD, so one wave's softmax work overlaps the other's matrix-core work):
//   WHICH = 0: S = Q K^T, P = exp2(S c - lse2), dV^T += dO^T P     (Q rows, dO^T, lse2 streamed)
//   WHICH = 1: S, dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS     (Q rows, dO rows, Q^T, lse2, D)
// S is recomputed by both (2 + 3 products instead of 4 in one kernel); each
// keeps its accumulator, K (and V) in registers and streams 64-query tiles
// through a 2-stage LDS ring.
// ===========================================================================
template <int D, int WHICH>
struct KvCfg {
    static constexpr int NW = 8;
    static constexpr int NT = 64 * NW;
    static constexpr int BK = 32 * NW;                   // keys per workgroup
    static constexpr int BQ = 64;                        // queries per tile
    static constexpr int RROW = 2 * D + 16;              // bytes per Q / dO row in LDS (padded)
    static constexpr int TROW = 2 * BQ + 16;             // bytes per dO^T / Q^T row in LDS (padded)
    static constexpr int RBYTES = dma_region_bytes(BQ * RROW);
    static constexpr int TBYTES = dma_region_bytes(D * TROW);
    static constexpr int NR = WHICH == 0 ? 1 : 2;        // row-major tiles: Q (and dO)
    static constexpr int VEC = BQ * 4;
    static constexpr int NV = WHICH == 0 ? 1 : 2;        // row vectors: lse2 (and D)
    static constexpr int STAGE = NR * RBYTES + TBYTES + NV * VEC;
    static constexpr int V_CHUNKS = NV * VEC / 16;
    static constexpr int QREGS = D / 16;
};

template <int D, bool CAUSAL, int WHICH>
__global__ __launch_bounds__(512) void bwd_kv_kernel(BParams p) {
    using C = KvCfg<D, WHICH>;
    constexpr int BK = C::BK, BQ = C::BQ, NT = C::NT;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int N = p.N;
    const int kt = blockIdx.x / p.BH;                    // causal: low key tiles see the most queries
    const int bh = blockIdx.x - kt * p.BH;
    const int k0 = kt * BK, kw0 = k0 + 32 * w, my_k = kw0 + l32;

    const size_t slice = static_cast<size_t>(bh) * N * D;
    const uint8_t* qg = p.q + slice * 2;
    const uint8_t* gg = p.dout + slice * 2;
    const uint8_t* tg = (WHICH == 0 ? p.dot : p.qt) + static_cast<size_t>(bh) * D * p.np * 2;
    const float* l2g = p.lse2 + static_cast<size_t>(bh) * N;
    const float* dsg = p.dsum + static_cast<size_t>(bh) * N;

    // K (and V) rows of this lane's key: B operands of S = Q K^T (and dP = dO V^T)
    u32x4 kf[C::QREGS], vf[WHICH == 1 ? C::QREGS : 1];
    {
        const bool ok = my_k < N;
        const size_t off = (slice + static_cast<size_t>(my_k) * D) * 2;
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i) {
            kf[i] = ok ? ld16(p.k + off + 2 * (16 * i + 8 * h)) : u32x4{0, 0, 0, 0};
            if constexpr (WHICH == 1) vf[i] = ok ? ld16(p.v + off + 2 * (16 * i + 8 * h)) : u32x4{0, 0, 0, 0};
        }
    }

    const int n_qt = (N + BQ - 1) / BQ;
    const int t0 = CAUSAL ? min(k0 / BQ, n_qt) : 0;
    const int t_first = CAUSAL ? max(t0, kw0 / BQ) : 0;  // first tile with a query at or after this wave's keys

    // Tiles go global -> LDS directly (buffer loads to LDS): a stage is Q rows
    // (and dO rows) at a 272-byte stride (16 granules + one pad), then the
    // transposed tile at 144 bytes (8 + 1), NB contiguous 1 KiB blocks, block b
    // copied by wave b mod 8; the hardware range check zero-fills rows past
    // the end of the sequence.  The row vectors (lse2, and D) follow through
    // registers: rows past the end get lse2 = +inf (P = 0) and D = 0.
    static_assert(C::RROW == 2 * D + 16 && C::TROW == 144, "LDS-DMA layout");
    constexpr int NB_R = C::RBYTES / 1024, NB = C::NR * NB_R + C::TBYTES / 1024, PER_W = (NB + 7) / 8;
    uint32_t doff[PER_W];
    int dn = 0;
#pragma unroll
    for (int i = 0; i < PER_W; ++i) {
        const int b = w + 8 * i;
        doff[i] = 0x40000000u;
        if (b < NB) {
            doff[i] = b < C::NR * NB_R ? dma_lane_offset(b % NB_R, lane, D / 8, D * 2, BQ)
                                       : dma_lane_offset(b - C::NR * NB_R, lane, BQ / 8, p.np * 2, D);
            dn = i + 1;
        }
    }
    const uint32_t smem_lds = lds_address(smem);
    auto copy_tile = [&](int t) {
        const int m0 = t * BQ;
        const uint32_t valid = static_cast<uint32_t>(min(N - m0, BQ)) * D * 2;
        const u32x4 rq = buffer_words(qg + static_cast<size_t>(m0) * D * 2, valid);
        const u32x4 rg = buffer_words(gg + static_cast<size_t>(m0) * D * 2, valid);
        const u32x4 rt = buffer_words(tg + static_cast<size_t>(m0) * 2, (static_cast<uint32_t>(D) * p.np - m0) * 2);
        const uint32_t stage = smem_lds + (t & 1) * C::STAGE;
#pragma unroll
        for (int i = 0; i < PER_W; ++i) {
            const int b = w + 8 * i;
            if (i < dn) {
                poison_block(stage + 1024 * b);
                lds_dma16(stage + 1024 * b, b < NB_R ? rq : (b < C::NR * NB_R ? rg : rt), doff[i]);
            }
        }
    };
    u32x4 vecst;
    auto load_vec = [&](int t) {
        if (tid < C::V_CHUNKS) {
            const int m0 = t * BQ;
            const int which = tid / (C::VEC / 16), r0 = m0 + 4 * (tid - which * (C::VEC / 16));
            const float* src = which == 0 ? l2g : dsg;
            const float fill = which == 0 ? __builtin_inff() : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) vecst[e] = __float_as_uint(r0 + e < N ? src[r0 + e] : fill);
        }
    };
    auto store_vec = [&](int t) {
        if (tid < C::V_CHUNKS)
            *reinterpret_cast<u32x4*>(smem + (t & 1) * C::STAGE + C::NR * C::RBYTES + C::TBYTES + 16 * tid) = vecst;
    };

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    // one 32-query block qb of tile t
    auto compute = [&](int t, int qb, bool masked) {
        const uint8_t* stage = smem + (t & 1) * C::STAGE;
        const uint8_t* qs = stage;
        const uint8_t* gs = stage + C::RBYTES;           // dO rows (dK only)
        const uint8_t* ts = stage + C::NR * C::RBYTES;
        const float* l2s = reinterpret_cast<const float*>(ts + C::TBYTES);
        const float* dss = l2s + BQ;
        const int rel = my_k - t * BQ - 32 * qb - 4 * h; // masked when rel > 8*(v/4) + v%4
        f32x16 s = {}, dp = {};
        const uint8_t* qr = qs + (32 * qb + l32) * C::RROW + 16 * h;
        const uint8_t* gr = gs + (32 * qb + l32) * C::RROW + 16 * h;
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ld16(qr + 32 * i)),
                                                       __builtin_bit_cast(bf16x8, kf[i]), s, 0, 0, 0);
            if constexpr (WHICH == 1)
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ld16(gr + 32 * i)),
                                                            __builtin_bit_cast(bf16x8, vf[i]), dp, 0, 0, 0);
        }
        float x[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(l2s + 32 * qb + 8 * g + 4 * h);
            f32x4 d4 = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (WHICH == 1) d4 = *reinterpret_cast<const f32x4*>(dss + 32 * qb + 8 * g + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = 4 * g + e;
                float pr = fast_exp2(fmaf(s[v], p.c_log2, -l4[e]));
                if (masked && CAUSAL && rel > 8 * g + e) pr = 0.0f;
                x[v] = WHICH == 0 ? pr : pr * (dp[v] - d4[e]);
            }
        }
        bf16x8 xf[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e) xf[cc][e] = static_cast<__bf16>(x[8 * cc + e]);
        const uint8_t* tr = ts + l32 * C::TROW + 16 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, ld16(tr + 32 * db * C::TROW + 32 * (2 * qb + cc))), xf[cc], acc[db], 0,
                    0, 0);
    };
    auto compute_block = [&](int t, int qb) {
        if (t < t_first) return;
        compute(t, qb, CAUSAL && t * BQ < kw0 + 31);
    };

    if (t0 < n_qt) {
        copy_tile(t0);
        load_vec(t0);
        store_vec(t0);
        wait_lds_dma();
    }
    __syncthreads();
    for (int t = t0; t < n_qt; ++t) {
        const bool more = t + 1 < n_qt;
        if (more) {
            copy_tile(t + 1);
            load_vec(t + 1);
        }
        compute_block(t, 0);
        compute_block(t, 1);
        if (more) {
            store_vec(t + 1);
            wait_lds_dma();
        }
        __syncthreads();
    }

    if (my_k < N) {
        uint8_t* out = (WHICH == 0 ? p.dv : p.dk) + (slice + static_cast<size_t>(my_k) * D) * 2;
        const float mul = WHICH == 0 ? 1.0f : p.scale;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = static_cast<__bf16>(acc[db][4 * g + e] * mul);
                *reinterpret_cast<bf16x4*>(out + 2 * (32 * db + 8 * g + 4 * h)) = ov;
            }
    }
}

// ===========================================================================
// dK and dV of d = 128 in one kernel, S computed once: the 8 waves form four
// pairs (w, w + 4) on one SIMD sharing 32 keys.  Wave w (group A) holds K and
// accumulates dV, wave w + 4 (group B) holds V and accumulates dK; they run
// the ping-pong one slot apart, so each SIMD holds one wave on its matrix
// cores while the other runs vector work.  Per 64-query tile t:
//   A: M_t = { dV^T += dO_{t-1}^T P_{t-1},  S_t = Q_t K^T }
//      V_t = { P_t = exp2(S c - lse2) (masked), to bf16, handed to B through LDS }
//   B: M_t = { dK^T += Q_{t-1}^T dS_{t-1},  dP_t = dO_t V^T }
//      V_t = { dS_t = P_t (dP - D) from A's bf16 P, to bf16 }
// A runs op k in slot k, B in slot k+1, so P_t is written in slot 2t+1 and
// read in slot 2t+2.  Row ring (3 stages): tile t's dO and Q rows, laid out
// with xr_granule so that S and dP read them as rows (slots 2t, 2t+1) and dV
// and dK through the transposing read (slots 2t+2, 2t+3); vector ring (3
// stages): lse2 and D, read in slots 2t+1, 2t+2.  Group B copies X_{j+2} and
// L_{j+2} in its vector slot 2j+2, into the stages tile j-1 left in slot 2j+1,
// and waits for them at the end of slot 2j+3.  Against the split dV and dK
// kernels this saves the dV kernel's S; dS is formed from the bf16 P (the
// value P*V sees) instead of the fp32 one.
// ===========================================================================
struct KvfCfg {
    static constexpr int D = 128, NW = 8, NT = 64 * NW, BK = 32 * NW / 2, BQ = 64, QB = BQ / 32;
    static constexpr int XREG = BQ * 256;                             // 16 KiB: dO rows, then Q rows
    static constexpr int X_BLOCKS = 2 * XREG / 1024;
    static constexpr int XSTAGE = X_BLOCKS * 1024, LSTAGE = 2 * 1024;
    static constexpr int PPAIR = 64 * 16 * 2 * QB;                    // bf16 P of one pair: 64 B a lane
    static constexpr int SMEM = 3 * XSTAGE + 3 * LSTAGE + 4 * PPAIR;
    static constexpr int QREGS = D / 16;
    static constexpr int AHEAD = 6;
};

template <bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_kvf_kernel(BParams p) {
    using C = KvfCfg;
    constexpr int D = C::D, BK = C::BK, BQ = C::BQ, QB = C::QB;
    static_assert(C::X_BLOCKS % 8 == 0 && C::SMEM <= 160 * 1024, "LDS layout");
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::SMEM];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, grp = w >> 2, h = lane >> 5, l32 = lane & 31;
    const int N = p.N;
    const int kt = blockIdx.x / p.BH;                    // causal: low key tiles see the most queries
    const int bh = blockIdx.x - kt * p.BH;
    const int k0 = kt * BK, kw0 = k0 + 32 * (w & 3), my_k = kw0 + l32;

    const size_t slice = static_cast<size_t>(bh) * N * D;
    const uint8_t* qg = p.q + slice * 2;
    const uint8_t* gg = p.dout + slice * 2;
    const float* l2g = p.lse2 + static_cast<size_t>(bh) * N;
    const float* dsg = p.dsum + static_cast<size_t>(bh) * N;

    // A: K rows of this lane's key (B operand of S = Q K^T); B: V rows (of dP = dO V^T)
    u32x4 bf[C::QREGS];
    {
        const bool ok = my_k < N;
        const uint8_t* src = (grp == 0 ? p.k : p.v) + (slice + static_cast<size_t>(my_k) * D) * 2;
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i) bf[i] = ok ? ld16(src + 2 * (16 * i + 8 * h)) : u32x4{0, 0, 0, 0};
    }

    // query tiles [t0, t0 + n_t) of the workgroup; this pair's work starts at local tile j_first
    const int n_qt = (N + BQ - 1) / BQ;
    const int t0 = CAUSAL ? min(k0 / BQ, n_qt) : 0;
    const int n_t = n_qt - t0;
    const int j_first = CAUSAL ? min(n_t, kw0 / BQ - t0) : 0;

    // ---- tile copies (group B, wave w & 3 copies blocks (w & 3) + 4i of a stage)
    const uint32_t smem_lds = lds_address(smem);
    const uint32_t xbase = smem_lds, lbase = xbase + 3 * C::XSTAGE;
    constexpr int X_PER_W = C::X_BLOCKS / 4;
    const uint32_t x_off = grp == 1 ? xr_copy_offset(w, lane) : 0u;
    auto copy_x = [&](int t) {                      // dO, Q rows of local tile t into X stage t % 3,
        const int m0 = (t0 + t) * BQ;                // its lse2 and D into L stage t % 3
        const uint32_t valid = static_cast<uint32_t>(min(N - m0, BQ));
        const u32x4 rg = buffer_words(gg + static_cast<size_t>(m0) * D * 2, valid * D * 2);
        const u32x4 rq = buffer_words(qg + static_cast<size_t>(m0) * D * 2, valid * D * 2);
        const uint32_t st = xbase + (t % 3) * C::XSTAGE + 1024 * (w & 3);
#pragma unroll
        for (int i = 0; i < X_PER_W; ++i) {
            poison_block(st + 4096 * i);
            lds_dma16(st + 4096 * i, i < X_PER_W / 2 ? rg : rq, x_off + 4096 * (i % (X_PER_W / 2)));
        }
        if ((w & 3) < 2) {
            const u32x4 rv = buffer_words((w & 3) == 0 ? l2g + m0 : dsg + m0, valid * 4);
            const uint32_t lb = lbase + (t % 3) * C::LSTAGE + 1024 * (w & 3);
            poison_block(lb);
            lds_dma16(lb, rv, lane < BQ / 4 ? 16u * lane : 0x40000000u);
        }
    };
    auto copies = [&](int j) {
        if (j + 2 < n_t) copy_x(j + 2);
    };

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    f32x16 s[QB];                                    // A: S; B: dP
    bf16x8 xf[2 * QB];                               // A: P; B: dS
    uint32_t lane_to[D / 32];                        // transposing reads of the X^T operand
#pragma unroll
    for (int db = 0; db < D / 32; ++db) lane_to[db] = xr_read_offset(lane, db);
    const int hi_delta = xr_hi_delta(lane);
    // row reads of S / dP's A operand (row l32 + 32 qb, granule 2i + h): xr_granule
    // depends on the row's low four bits only, so qb adds a constant
    const int xr_row = l32 * 256, xr_fl = 4 * (l32 & 3) + ((l32 >> 2) & 3);
    uint8_t* pex = smem + 3 * C::XSTAGE + 3 * C::LSTAGE + (w & 3) * C::PPAIR + 16 * lane;

    // A: S = Q_t K^T; B: dP = dO_t V^T (local tile j, 32-query blocks qb)
    auto op_s = [&](int j) {
        // A: Q rows (second half of the stage); B: dO rows (first half)
        const uint8_t* rr = smem + (j % 3) * C::XSTAGE + (1 - grp) * C::XREG + xr_row;
        bf16x8 a[QB * C::QREGS];
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                a[QB * i + qb] = __builtin_bit_cast(bf16x8, ld16(rr + 32 * qb * 256 + 16 * ((2 * i + h) ^ xr_fl)));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[QB * i + qb], __builtin_bit_cast(bf16x8, bf[i]), s[qb],
                                                               0, 0, 0);
        pipeline_lds_mfma<QB * C::QREGS, C::AHEAD>();
    };
    // A: P of local tile j (query of register v of block qb: (t0 + j) BQ + 32 qb +
    // acc_row(v, h)), 0 before the key (causal, masked) or past N (ragged)
    auto op_v_a = [&](int j, bool masked, bool ragged) {
        const float* l2s = reinterpret_cast<const float*>(smem + 3 * C::XSTAGE + (j % 3) * C::LSTAGE);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int rel = my_k - (t0 + j) * BQ - 32 * qb - 4 * h;   // masked when rel > 8*(v/4) + v%4
            const int lim = N - 1 - ((t0 + j) * BQ + 32 * qb + 4 * h);  // ragged: past N when 8*(v/4) + v%4 > lim
            float x[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(l2s + 32 * qb + 8 * g + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float pr = fast_exp2(fmaf(s[qb][4 * g + e], p.c_log2, -l4[e]));
                    if ((masked && rel > 8 * g + e) || (ragged && 8 * g + e > lim)) pr = 0.0f;
                    x[4 * g + e] = pr;
                }
            }
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[2 * qb + cc][e] = static_cast<__bf16>(x[8 * cc + e]);
                *reinterpret_cast<u32x4*>(pex + 1024 * (2 * qb + cc)) = __builtin_bit_cast(u32x4, xf[2 * qb + cc]);
            }
        }
    };
    // B: dS = P (dP - D) of local tile j, P as A wrote it
    auto op_v_b = [&](int j) {
        const float* dss = reinterpret_cast<const float*>(smem + 3 * C::XSTAGE + (j % 3) * C::LSTAGE + 1024);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            bf16x8 pb[2];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) pb[cc] = __builtin_bit_cast(bf16x8, ld16(pex + 1024 * (2 * qb + cc)));
            float x[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(dss + 32 * qb + 8 * g + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = 4 * g + e;
                    x[v] = static_cast<float>(pb[v >> 3][v & 7]) * (s[qb][v] - d4[e]);
                }
            }
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[2 * qb + cc][e] = static_cast<__bf16>(x[8 * cc + e]);
        }
    };
    // A: dV^T += dO^T P; B: dK^T += Q^T dS (local tile j)
    auto op_acc = [&](int j) {
        const lds_u8* ts = (const lds_u8*)smem + (j % 3) * C::XSTAGE + grp * C::XREG;
        constexpr int NC = 2 * QB;                      // 16-query chunks of the tile
        bf16x8 a[NC * (D / 32)];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) {
                const i16x4 lo = ds_read_tr16(ts + lane_to[db] + 16 * cc * 256);
                const i16x4 hi = ds_read_tr16(ts + lane_to[db] + hi_delta + 16 * cc * 256);
                a[NC * db + cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int cc = 0; cc < NC; ++cc)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[NC * db + cc], xf[cc], acc[db], 0, 0, 0);
        pipeline_lds_mfma<NC * (D / 32), C::AHEAD, 2>();
    };
    auto masked_tile = [&](int j) { return CAUSAL && (t0 + j) * BQ < kw0 + 31; };
    auto ragged_tile = [&](int j) { return (t0 + j) * BQ + BQ > N; };
    auto slot_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: group B copies X_0, L_0 and waits; everyone meets at barrier 0
    if (grp == 1 && n_t > 0) {
        copy_x(0);
        wait_lds_dma();
    }
    lds_barrier();

    if (n_t > 0) {
        if (grp == 0) {
            // A: M_0 | V_0 M_1 | ... | V_{n-1} M_n | idle, from local tile j_first on
            for (int j = 0; j < j_first; ++j) {
                slot_end();
                slot_end();
            }
            if (j_first < n_t) {
                op_s(j_first);
                slot_end();
                op_v_a(j_first, masked_tile(j_first), ragged_tile(j_first));
                slot_end();
                for (int j = j_first; j + 1 < n_t; ++j) {
                    op_acc(j);
                    __builtin_amdgcn_sched_barrier(0);
                    op_s(j + 1);
                    slot_end();
                    op_v_a(j + 1, false, ragged_tile(j + 1));
                    slot_end();
                }
                op_acc(n_t - 1);
            }
            slot_end();
            slot_end();
        } else {
            // B: copies | M_0 | V_0 + copies, M_1 | ... | V_{n-1} + copies, M_n
            if (1 < n_t) copy_x(1);
            slot_end();
            for (int j = 0; j < j_first; ++j) {
                wait_lds_dma();
                slot_end();
                copies(j);
                slot_end();
            }
            if (j_first < n_t) {
                op_s(j_first);
                wait_lds_dma();
                slot_end();
                op_v_b(j_first);
                copies(j_first);
                slot_end();
                for (int j = j_first; j + 1 < n_t; ++j) {
                    op_acc(j);
                    __builtin_amdgcn_sched_barrier(0);
                    op_s(j + 1);
                    wait_lds_dma();
                    slot_end();
                    op_v_b(j + 1);
                    copies(j + 1);
                    slot_end();
                }
                op_acc(n_t - 1);
            }
            wait_lds_dma();
            slot_end();
        }
    }

    if (my_k < N) {
        uint8_t* out = (grp == 0 ? p.dv : p.dk) + (slice + static_cast<size_t>(my_k) * D) * 2;
        const float mul = grp == 0 ? 1.0f : p.scale;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = static_cast<__bf16>(acc[db][4 * g + e] * mul);
                *reinterpret_cast<bf16x4*>(out + 2 * (32 * db + 8 * g + 4 * h)) = ov;
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_d(BParams bp, const void* o, const float* lse, float* lse2, float* dsum, hipStream_t st) {
    const long long rows = static_cast<long long>(bp.BH) * bp.N;
    const long long pgrid = (rows * (D / 8) + 255) / 256;
    if (pgrid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(static_cast<int>(pgrid)), dim3(256), 0, st,
                       static_cast<const uint8_t*>(o), bp.dout, lse, lse2, dsum, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    BParams a = bp;
    a.n_tiles = (bp.N + DqCfg<D>::BM - 1) / DqCfg<D>::BM;
    const long long g1 = static_cast<long long>(a.n_tiles) * bp.BH;
    BParams b = bp;
    b.n_tiles = (bp.N + KvCfg<D, 0>::BK - 1) / KvCfg<D, 0>::BK;
    const long long g2 = static_cast<long long>(b.n_tiles) * bp.BH;
    if (g1 > 0x7FFFFFFFLL || g2 > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    if constexpr (D == 128) {
        BParams f = bp;
        f.n_tiles = (bp.N + KvfCfg::BK - 1) / KvfCfg::BK;
        const long long g3 = static_cast<long long>(f.n_tiles) * bp.BH;
        if (g3 > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd_kvf_kernel<CAUSAL>), dim3(static_cast<int>(g3)), dim3(KvfCfg::NT), 0, st, f);
    } else {
        hipLaunchKernelGGL((bwd_kv_kernel<D, CAUSAL, 0>), dim3(static_cast<int>(g2)), dim3(KvCfg<D, 0>::NT), 0, st, b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_kv_kernel<D, CAUSAL, 1>), dim3(static_cast<int>(g2)), dim3(KvCfg<D, 1>::NT), 0, st, b);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if constexpr (D == 128) {
        hipLaunchKernelGGL((bwd_dq_pp_kernel<CAUSAL, kDqSlotKeys>), dim3(static_cast<int>(g1)), dim3(DqPPCfg<kDqSlotKeys>::NT),
                           0, st, a);
    } else {
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(static_cast<int>(g1)), dim3(DqCfg<D>::NT), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    BParams bp;
    bp.q = static_cast<const uint8_t*>(a.q);
    bp.k = static_cast<const uint8_t*>(a.k);
    bp.v = static_cast<const uint8_t*>(a.v);
    bp.dout = static_cast<const uint8_t*>(a.dout);
    bp.qt = static_cast<const uint8_t*>(a.qt);
    bp.dot = static_cast<const uint8_t*>(a.dot);
    bp.kt = static_cast<const uint8_t*>(a.kt);
    bp.lse2 = a.lse2;
    bp.dsum = a.dsum;
    bp.dq = static_cast<uint8_t*>(a.dq);
    bp.dk = static_cast<uint8_t*>(a.dk);
    bp.dv = static_cast<uint8_t*>(a.dv);
    bp.BH = a.BH;
    bp.N = a.N;
    bp.np = a.np;
    bp.n_tiles = 0;
    bp.c_log2 = a.softmax_scale * kLog2e;
    bp.scale = a.softmax_scale;
    switch (a.d) {
        case 32: return a.causal ? launch_bwd_d<32, true>(bp, a.o, a.lse, a.lse2, a.dsum, stream)
                                 : launch_bwd_d<32, false>(bp, a.o, a.lse, a.lse2, a.dsum, stream);
        case 64: return a.causal ? launch_bwd_d<64, true>(bp, a.o, a.lse, a.lse2, a.dsum, stream)
                                 : launch_bwd_d<64, false>(bp, a.o, a.lse, a.lse2, a.dsum, stream);
        case 128: return a.causal ? launch_bwd_d<128, true>(bp, a.o, a.lse, a.lse2, a.dsum, stream)
                                  : launch_bwd_d<128, false>(bp, a.o, a.lse, a.lse2, a.dsum, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
