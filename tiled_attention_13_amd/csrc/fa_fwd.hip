// Fused attention forward for gfx950 (MI355X): O = softmax(scale * Q K^T) V and lse.
//
// A workgroup owns a tile of queries of one (batch, head) and walks the
// key/value sequence in 64-key tiles: the tiled double loop of "Core
// principles behind FlashAttention's speed-up" (section 1.1) in the
// FlashAttention-2 order, parallel over batch, heads and query tiles (the
// "Flash Attention" tag page, excerpt on V2).  Everything between loading a
// K/V tile and writing O stays in registers and LDS (same page, section 1.2).
//
// Scores are produced transposed, S^T = K Q^T, on 32x32 MFMAs: A = 32 keys
// from LDS, B = 32 queries held in registers for the whole loop.  In the
// 32x32 accumulator layout lane l owns column l % 32, so every lane holds 16
// scores of ONE query (the other 16 of each 32-key block sit in lane l ^ 32).
// Row reductions are in-lane plus one v_permlane32_swap, and the
// probabilities already sit where the B operand of O^T += V^T P^T wants
// them: P never goes through LDS.  V tiles sit in LDS as they are in memory
// (key rows, 16-byte granules XOR-swizzled per row) and the V^T operand of
// that product is gathered with gfx950's transposing LDS read
// (ds_read_b64_tr_b16), so no transposed copy of V is ever made.
//
// Online softmax (Triton walkthrough page, section 2.1): running max m and
// running sum l per query, kept in base-2 units with softmax_scale*log2(e)
// folded into one FMA before v_exp_f32; the accumulator is rescaled by
// exp2(m_old - m_new) and the division by l is deferred to the epilogue (tag
// page, excerpt on V2).  l is summed from the fp32 probabilities before they
// are rounded to bf16.
//
// Causal (Triton walkthrough page, section 3.1): key tiles entirely above
// the diagonal are never loaded, a wave skips tiles above its own rows, and
// only the tile that crosses the diagonal (or the sequence end) compares
// indices.  Workgroups are issued heaviest query tile first.
//
// FP8 (same page, section 4.1): Q and K arrive as e4m3fn codes with one
// fp32 scale per 64-row tile; S^T runs on the 32x32x64 f8f6f4 MFMA (32x32x16
// fp8 for d = 32) and the dequantisation 1/(q_scale*k_scale) is folded into
// the exp2 constant (64-key tiles keep one K scale per tile).  V and P*V stay
// bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

struct KParams {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    const uint8_t* vt;      // V^T [BH, D, np] with tile-permuted keys (bf16/FP8 kernel)
    uint8_t* o;
    float* lse;
    const float* q_scale;
    const float* k_scale;
    int BH;
    int N;
    int np;
    int n_qtiles;
    float c_log2;       // softmax_scale * log2(e)
    // partial results over key ranges (PARTIAL kernels only)
    float* o32;         // [n_splits, BH, N, D] normalised over the split's keys
    float* lse_part;    // [n_splits, BH, N], -inf where the split has no visible key
    int kt_lo, kt_hi;   // key tiles [kt_lo, kt_hi) of the launch
    int tps;            // key tiles per split
    int n_splits;
    // block-sparse kernels: per (bh, query tile) the list of key tiles to visit,
    // entry = tile | (bit b set if 64-query block b of the tile needs it) << 24
    const uint32_t* bs_list;
    const int* bs_count;
    int bs_stride;
    // FP8 P*V: MFMA block-scale bytes (127 - e) of the e4m3 V^T, [BH, n_tiles, D]
    const uint8_t* vscale;
    // d = 128 kernel: heads per band of the XCD-banded work order (0: query-tile major)
    int band;
};

// Number of XCDs: consecutive workgroups of a launch go to the eight XCDs in
// turn, each with its own L2.
constexpr int kXcds = 8;

// a float in the constant address space: loads through it with a wave-uniform
// address become scalar loads (the data is written before the kernel starts)
typedef __attribute__((address_space(4))) const float const_f32;

// kernel variants of fwd_pp_kernel
enum : int { kModeDense = 0, kModePartial = 1, kModeSparse = 2 };

// ---------------------------------------------------------------------------
// Online-softmax step on the scores one lane holds for its query.
// s[NS]: scores (already masked to -inf), c: scale into base-2 units.
// Updates m (base-2 reference max) and l (this lane's part of the running
// sum), overwrites s with the probabilities and returns the factor alpha by
// which the partial O must be rescaled.
//
// The reference max only moves when the tile's max exceeds it by more than
// kRescaleSlack (base-2 units).  Softmax is invariant to the reference, so
// the result is the same; probabilities are then bounded by 2^kRescaleSlack
// instead of 1, and most tiles need no rescale.  bf16 and fp32 keep their
// relative precision at any exponent; the range bound is the fp32 P*V sum,
// at most N * 2^45 * max|v|, which stays finite for N * max|v| < 2^82.  (The
// FP8 P*V path rescales P into the e4m3 range per tile, so it sees the same
// bound.)  A wide slack matters where a few keys score far above the rest:
// each new maximum would otherwise cost a rescale of the 64 O accumulators.
// ---------------------------------------------------------------------------
constexpr float kRescaleSlack = 45.0f;
constexpr float kRescaleBound = 0x1p45f;     // 2^kRescaleSlack

template <int NS>
__device__ __forceinline__ float softmax_step(float (&s)[NS], float c, float& m, float& l) {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < NS; ++i) mx = fmaxf(mx, s[i]);
    const float mx2 = max_halves(mx) * c;
    float alpha = 1.0f;
    if (mx2 > m + kRescaleSlack) {        // also taken on the first unmasked tile (m = -inf)
        alpha = fast_exp2(m - mx2);
        m = mx2;
    }
    const float m_use = (m == kNegInf) ? 0.0f : m;   // nothing unmasked yet: all p are 0
    float rs = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const float p = fast_exp2(fmaf(s[i], c, -m_use));
        s[i] = p;
        rs += p;
    }
    l = fmaf(l, alpha, rs);
    return alpha;
}

// The same step for NS scores whose first and second halves are scaled into
// base-2 units by different factors (c0, c1 > 0): the two 64-key halves of an
// FP8 tile, each with its own K scale.
template <int NS>
__device__ __forceinline__ float softmax_step2(float (&s)[NS], float c0, float c1, float& m, float& l) {
    float ma = kNegInf, mb = kNegInf;
#pragma unroll
    for (int i = 0; i < NS / 2; ++i) ma = fmaxf(ma, s[i]);
#pragma unroll
    for (int i = NS / 2; i < NS; ++i) mb = fmaxf(mb, s[i]);
    const float mx2 = fmaxf(max_halves(ma) * c0, max_halves(mb) * c1);
    float alpha = 1.0f;
    if (mx2 > m + kRescaleSlack) {        // also taken on the first unmasked tile (m = -inf)
        alpha = fast_exp2(m - mx2);
        m = mx2;
    }
    const float m_use = (m == kNegInf) ? 0.0f : m;   // nothing unmasked yet: all p are 0
    float rs = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const float p = fast_exp2(fmaf(s[i], i < NS / 2 ? c0 : c1, -m_use));
        s[i] = p;
        rs += p;
    }
    l = fmaf(l, alpha, rs);
    return alpha;
}

// Probabilities against the current reference m alone, without the row max:
// the first NS/2 scores scaled by c0, the rest by c1, packed to bf16 into pf,
// their sum added to l.  Taken only when every lane's part of the sum is at
// most 2^kRescaleSlack: then so is every probability, and softmax_step(2)
// would have left the reference where it is and computed the same values in
// the same order.  Otherwise (a new maximum far above the reference; an inf
// or NaN score; m = -inf) it returns false for the whole wave, leaving l and
// the scores as they were (pf undefined): the caller then takes the full step.
template <int NS>
__device__ __forceinline__ bool softmax_at_ref(const float (&s)[NS], float c0, float c1, float m, float& l,
                                               bf16x8 (&pf)[NS / 8]) {
    float rs = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; i += 2) {
        const float p0 = fast_exp2(fmaf(s[i], i < NS / 2 ? c0 : c1, -m));
        const float p1 = fast_exp2(fmaf(s[i + 1], i + 1 < NS / 2 ? c0 : c1, -m));
        rs += p0;
        rs += p1;
        pf[i / 8][i % 8] = static_cast<__bf16>(p0);
        pf[i / 8][i % 8 + 1] = static_cast<__bf16>(p1);
    }
    // The packs stay ahead of the test: sunk past it (pf is only used when it
    // passes), they would keep every probability live across it, next to the
    // scores the fallback needs (measured: 12 to 28 VGPRs fewer; d = 32 -1 %).
#pragma unroll
    for (int c = 0; c < NS / 8; ++c) asm volatile("" : : "v"(pf[c]));
    if (__builtin_amdgcn_ballot_w64(!(rs <= kRescaleBound)) != 0) return false;
    l += rs;
    return true;
}

// Same step for an e4m3 P*V product: the probabilities come out multiplied by
// 2^f, with f the largest integer (at most 127) for which this tile's largest
// probability stays within the e4m3 range 448 (so they fill that range before
// rounding); 127 - f is the matrix core's block exponent that undoes it.  l
// still sums the unscaled fp32 probabilities.
template <int NS>
__device__ __forceinline__ float softmax_step_p8(float (&s)[NS], float c, float& m, float& l, int& scale_b) {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < NS; ++i) mx = fmaxf(mx, s[i]);
    const float mx2 = max_halves(mx) * c;
    float alpha = 1.0f;
    if (mx2 > m + kRescaleSlack) {
        alpha = fast_exp2(m - mx2);
        m = mx2;
    }
    const float m_use = (m == kNegInf) ? 0.0f : m;
    // log2 of the tile's largest probability is mx2 - m_use; log2(448) = 8.807...
    const float fl = floorf(8.807354922f - (mx2 - m_use));
    const int f = fl > 126.0f ? 126 : (fl < -126.0f ? -126 : static_cast<int>(fl));   // -inf tile: 126
    const float shift = static_cast<float>(f) - m_use;
    float rs = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const float p = fast_exp2(fmaf(s[i], c, shift));
        s[i] = p;
        rs += p;
    }
    l = fmaf(rs, __int_as_float((127 - f) << 23), l * alpha);      // rs * 2^-f
    scale_b = 127 - f;
    return alpha;
}

// The same for a 128-key tile as two 64-key halves, each a scale tile of its
// own (the first NS/2 scores scaled into base-2 units by c0, the rest by c1):
// one reference for the tile, one 2^f per half, scale_b[h] = 127 - f of half h.
template <int NS>
__device__ __forceinline__ float softmax_step_p8x2(float (&s)[NS], float c0, float c1, float& m, float& l,
                                                   int (&scale_b)[2]) {
    float ma = kNegInf, mb = kNegInf;
#pragma unroll
    for (int i = 0; i < NS / 2; ++i) ma = fmaxf(ma, s[i]);
#pragma unroll
    for (int i = NS / 2; i < NS; ++i) mb = fmaxf(mb, s[i]);
    const float ha = max_halves(ma) * c0, hb = max_halves(mb) * c1;
    const float mx2 = fmaxf(ha, hb);
    float alpha = 1.0f;
    if (mx2 > m + kRescaleSlack) {
        alpha = fast_exp2(m - mx2);
        m = mx2;
    }
    const float m_use = (m == kNegInf) ? 0.0f : m;
    l *= alpha;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const float fl = floorf(8.807354922f - ((hf ? hb : ha) - m_use));
        const int f = fl > 126.0f ? 126 : (fl < -126.0f ? -126 : static_cast<int>(fl));   // -inf half: 126
        const float shift = static_cast<float>(f) - m_use, c = hf ? c1 : c0;
        float rs = 0.0f;
#pragma unroll
        for (int i = hf * NS / 2; i < (hf + 1) * NS / 2; ++i) {
            const float pr = fast_exp2(fmaf(s[i], c, shift));
            s[i] = pr;
            rs += pr;
        }
        l = fmaf(rs, __int_as_float((127 - f) << 23), l);      // rs * 2^-f
        scale_b[hf] = 127 - f;
    }
    return alpha;
}

// 16-byte granule of a bf16 V key row in LDS: data granule g of key row `row`
// sits at granule v_granule<D>(row, g), an XOR and so its own inverse.  The
// transposing reads of the P*V operand take, per 32 lanes, four consecutive
// key rows x 64 bytes (32 head dims); the swizzle puts those four pieces on
// four distinct quarters of the 64 LDS banks.
template <int D>
__device__ __forceinline__ int v_granule(int row, int g) {
    if constexpr (D == 128) return g ^ (4 * (row & 3));
    else if constexpr (D == 64) return g ^ (4 * ((row >> 1) & 1));
    else return g;
}

// Byte position, inside a 64-key row of the e4m3 V^T, of key kk: the order in
// which one lane's 32 P values (the two 32-key score blocks of its query, in
// register order) meet the k-slots of the 32x32x64 e4m3 MFMA.
__device__ __forceinline__ int f8_slot(int kk) {
    return (((kk >> 2) & 1) << 5) | (((kk >> 5) & 1) << 4) | (((kk >> 3) & 3) << 2) | (kk & 3);
}

// ===========================================================================
// bf16 / fp8 kernel, ping-pong schedule
//
// 8 waves, 256 queries per workgroup (32 per wave), 64-key tiles shared by all
// eight waves through a 3-stage LDS ring.  Waves 0-3 (group A) and 4-7
// (group B) sit one per SIMD each and run half a tile apart: every barrier
// ends a "slot" in which one group issues the matrix-core work of a tile
// (O^T += V^T P^T for the previous tile, then S^T = K Q^T for this one) while
// the other runs the softmax, rescale and tile copy on the vector ALUs, so
// each SIMD always has MFMA work from one wave to overlap the other's VALU.
//
// Per wave the op sequence is M_0 V_0 M_1 V_1 ... V_{n-1} M_n with
//   M_j = { PV_{j-1}, S_j }   (matrix cores)
//   V_j = { softmax_j, rescale, publish a staged tile, prefetch the next }
// group A runs op k in slot k, group B in slot k+1.  Tile t lives in LDS
// buffer t % 3.  A writes its half of tile t in V_{t-1} (slot 2t-1), B in
// V_{t-2} (slot 2t-2); the last reader of the previous occupant (B's PV in
// slot 2t-3) is done by then, and A first reads tile t in slot 2t.  Global
// loads land in registers two slots before they are written to LDS.
// ===========================================================================

template <int D, bool CAUSAL, bool FP8, bool PV8 = false, int MODE = kModeDense>
struct PPCfg {
    static constexpr int NW = 8;
    static constexpr int NT = 64 * NW;
    static constexpr int BM = 32 * NW;           // queries per workgroup
    static constexpr int BN = kKeyTile;          // keys per tile
    // K and V tiles go global -> LDS directly (buffer loads to LDS), issued a
    // slot earlier than a register copy would store them, so the ring has a
    // fourth stage.  Not in the block-sparse kernel (its short runs of listed
    // tiles measured slower that way), nor for the e4m3 V^T at d = 32 (its
    // 2.5 KiB tile is not a whole number of 1 KiB copy blocks).
    static constexpr bool DMA = MODE != kModeSparse && !(PV8 && D == 32);
    static constexpr int STAGES = DMA ? 4 : 3;
    static constexpr int ES = FP8 ? 1 : 2;       // bytes per Q/K element
    static constexpr int KROW = D * ES + 16;     // bytes per K row in LDS (padded)
    static constexpr int VES = PV8 ? 1 : 2;      // bytes per V element
    // bf16 V: BN key rows of D*2 bytes, granules swizzled (v_granule); e4m3 V
    // (FP8 P*V): D rows of V^T, BN keys each plus 16 bytes of padding
    static constexpr int VROW = PV8 ? VES * BN + 16 : D * 2;
    static constexpr int KBYTES = BN * KROW;
    static constexpr int VBYTES = PV8 ? D * VROW : BN * VROW;
    static constexpr int SBYTES = PV8 ? (D + 15) / 16 * 16 : 0;   // V block exponents of the tile
    static constexpr int STAGE = KBYTES + VBYTES + SBYTES;
    static constexpr int K_CPR = D * ES / 16;    // 16-byte chunks per K row
    static constexpr int K_CHUNKS = BN * K_CPR;
    static constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
    static constexpr int V_CPR = PV8 ? BN / 16 : D * 2 / 16;       // 16-byte chunks per V (e4m3 V^T) row
    static constexpr int V_CHUNKS = PV8 ? D * V_CPR : BN * V_CPR;    // 16-byte chunks of a V tile
    static constexpr int V_PER_T = (V_CHUNKS + NT - 1) / NT;
    static constexpr bool F8W = FP8 && (D % 64 == 0);
    static constexpr bool F8N = FP8 && !F8W;
    static constexpr int QREGS = F8W ? D / 64 : D / 16;
};

// The dense d = 32 kernel (FP8; bf16 at d = 32 has a kernel of its own) asks
// for 128 VGPRs (four waves per SIMD: two workgroups per CU); the others keep
// the wider budget, which they need (at d = 64 the transposing V reads take
// the dense kernel past 128).
template <int D, bool CAUSAL, bool FP8, int MODE, bool PV8 = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu((D == 32 && MODE == kModeDense) ? 4 : 2)))
void fwd_pp_kernel(KParams p) {
    using C = PPCfg<D, CAUSAL, FP8, PV8, MODE>;
    constexpr bool PARTIAL = MODE == kModePartial, SPARSE = MODE == kModeSparse;
    constexpr int BM = C::BM, BN = C::BN, NT = C::NT, ES = C::ES;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::STAGES * C::STAGE];

    const int tid = threadIdx.x;
    // wave index as a scalar, so every per-wave decision below is a uniform branch
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, grp = w >> 2, h = lane >> 5, l32 = lane & 31;
    const int N = p.N;

    int qt = blockIdx.x / p.BH;
    const int bh = blockIdx.x - qt * p.BH;
    int split = 0;
    if (PARTIAL) {
        split = qt / p.n_qtiles;
        qt -= split * p.n_qtiles;
    }
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;        // heaviest query tiles first
    const int q0 = qt * BM;
    const int qw0 = q0 + 32 * w;
    const int my_q = qw0 + l32;

    const size_t slice = static_cast<size_t>(bh) * N * D;
    const uint8_t* qg = p.q + slice * ES;
    const uint8_t* kg = p.k + slice * ES;
    // V of this (b, h): [N, D] bf16 rows, or (FP8 P*V) the e4m3 V^T, D rows of np keys
    const uint8_t* vg = PV8 ? p.vt + static_cast<size_t>(bh) * D * p.np : p.v + slice * 2;

    // ---- Q fragments (B operand of S^T = K Q^T)
    u32x4 qf[C::F8W ? 2 * C::QREGS : C::QREGS];
    {
        const bool ok = my_q < N;
        const uint8_t* row = qg + static_cast<size_t>(my_q) * D * ES;
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i) {
            if constexpr (C::F8W) {
                qf[2 * i] = ok ? ld16(row + 64 * i + 32 * h) : u32x4{0, 0, 0, 0};
                qf[2 * i + 1] = ok ? ld16(row + 64 * i + 32 * h + 16) : u32x4{0, 0, 0, 0};
            } else if constexpr (C::F8N) {
                const u32x2 x = ok ? *reinterpret_cast<const u32x2*>(row + 16 * i + 8 * h) : u32x2{0, 0};
                qf[i] = u32x4{x[0], x[1], 0, 0};
            } else {
                qf[i] = ok ? ld16(row + 2 * (16 * i + 8 * h)) : u32x4{0, 0, 0, 0};
            }
        }
    }

    const int n_scale = (N + 63) / 64;
    float c_q = p.c_log2;
    if (FP8) c_q = p.c_log2 / p.q_scale[bh * n_scale + (qw0 < N ? qw0 : N - 1) / 64];

    // key tiles [lo, lo + n_kt) of this workgroup; tiles are counted from lo below
    const int n_all = (N + BN - 1) / BN;
    int lo = 0, hi = n_all;
    if (PARTIAL) {
        lo = p.kt_lo + split * p.tps;
        hi = min(p.kt_hi, lo + p.tps);
    }
    if (CAUSAL) hi = min(hi, (min(q0 + BM, N) + BN - 1) / BN);
    const uint32_t* bs = nullptr;
    if (SPARSE) {
        bs = p.bs_list + static_cast<size_t>(bh * p.n_qtiles + qt) * p.bs_stride;
        hi = p.bs_count[bh * p.n_qtiles + qt];
    }
    const int n_kt = hi - lo;
    // key tile of list position t, and whether this wave computes it
    auto tile_of = [&](int t) -> int { return SPARSE ? static_cast<int>(bs[t] & 0xFFFFFFu) : lo + t; };
    auto needs = [&](int t) -> bool {
        return ((bs[t] >> (24 + (w >> 1))) & 1u) != 0 && !(CAUSAL && tile_of(t) * BN > qw0 + 31);
    };
    // last key tile with any key at or before this wave's last query
    // (negative when a key range lies entirely after this wave's queries)
    const int j_last = CAUSAL ? min(n_kt - 1, (qw0 + 31) / BN - lo) : n_kt - 1;

    if (SPARSE && n_kt <= 0) {                    // the block table leaves these queries no key
        if (my_q < N) {
            uint8_t* orow = p.o + (slice + static_cast<size_t>(my_q) * D) * 2;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<u32x2*>(orow + 2 * (32 * db + 8 * g + 4 * h)) = u32x2{0u, 0u};
            if (p.lse != nullptr && h == 0) p.lse[static_cast<size_t>(bh) * N + my_q] = kNegInf;
        }
        return;
    }
    if (PARTIAL && n_kt <= 0) {                   // no key of the range is visible to any query here
        if (my_q < N) {
            const size_t row = (static_cast<size_t>(split) * p.BH + bh) * N + my_q;
            float* orow = p.o32 + row * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * h) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (h == 0) p.lse_part[row] = kNegInf;
        }
        return;
    }

    // ---- global -> register staging of this thread's share of one K/V tile
    u32x4 kst[C::K_PER_T];
    u32x4 vst[C::V_PER_T];
    u32x4 sst = {0, 0, 0, 0};                    // FP8 P*V: V block exponents of the tile
    const int n_all_tiles = (N + BN - 1) / BN;
    // Tile copies go through buffer loads: the tile's base and the number of
    // valid bytes live in scalar registers, each thread's offset within the tile
    // is fixed, and rows past the end of the sequence read as zero (the hardware
    // range check), so full and partial tiles share one path.
    // DMA path: a stage is BN K rows (KROW-byte stride: D*ES/16 granules of 16
    // bytes + one pad granule) then the V tile (BN key rows of D*2 bytes with
    // swizzled granules; FP8 P*V: D e4m3 V^T rows, BN/16 granules + one pad),
    // i.e. DMA_ALL contiguous 1 KiB blocks, one LDS-DMA instruction each; group
    // A copies the first DMA_A blocks, group B the rest, block b of a group by
    // its wave b mod 4.  Each lane's source offset is chosen so that its 16
    // bytes land where the layout wants them; a lane that falls on a pad
    // granule reads past the buffer (zero, no memory traffic).  The FP8 P*V
    // block exponents after them still go through registers.
    constexpr int DMA_K = C::KBYTES / 1024, DMA_ALL = (C::KBYTES + C::VBYTES) / 1024;
    constexpr int DMA_A = (DMA_ALL + 1) / 2, DMA_PER_W = (DMA_A + 3) / 4;
    constexpr int KG = C::KROW / 16, KD = D * ES / 16, VG = C::VROW / 16, VD = BN * C::VES / 16;
    uint32_t dma_off[DMA_PER_W];
    int dma_n = 0;
    uint32_t smem_lds = 0;
    if constexpr (C::DMA) {
        static_assert(C::KBYTES % 1024 == 0 && C::VBYTES % 1024 == 0 && KG == KD + 1 && (!PV8 || VG == VD + 1),
                      "LDS-DMA layout");
        smem_lds = static_cast<uint32_t>(reinterpret_cast<size_t>((__attribute__((address_space(3))) uint8_t*)smem));
        const int b0 = grp == 0 ? 0 : DMA_A, b1 = grp == 0 ? DMA_A : DMA_ALL;
#pragma unroll
        for (int i = 0; i < DMA_PER_W; ++i) {
            const int b = b0 + (w & 3) + 4 * i;
            uint32_t off = 0x40000000u;
            if (b < b1) {
                if (b < DMA_K) {
                    const int g = 64 * b + lane, row = g / KG, col = g - KG * row;
                    if (col < KD) off = row * (D * ES) + 16 * col;
                } else if constexpr (PV8) {
                    const int g = 64 * (b - DMA_K) + lane, row = g / VG, col = g - VG * row;
                    if (col < VD) off = static_cast<uint32_t>(row) * p.np + 16 * col;
                } else {
                    // LDS granule pos of key row `row` holds V granule v_granule<D>(row, pos)
                    const int g = 64 * (b - DMA_K) + lane, row = g / VG, pos = g - VG * row;
                    off = row * (D * 2) + 16 * v_granule<D>(row, pos);
                }
                dma_n = i + 1;
            }
            dma_off[i] = off;
        }
    }
    auto dma_tile = [&](int t) {
        const int n0 = tile_of(t) * BN;
        const uint64_t ka = reinterpret_cast<uint64_t>(kg + static_cast<size_t>(n0) * D * ES);
        const uint64_t va = reinterpret_cast<uint64_t>(PV8 ? vg + n0 : vg + static_cast<size_t>(n0) * D * 2);
        const u32x4 kr = {static_cast<uint32_t>(ka), static_cast<uint32_t>(ka >> 32) & 0xFFFFu,
                          static_cast<uint32_t>(min(N - n0, BN) * D * ES), static_cast<uint32_t>(kBufferFlags)};
        const u32x4 vr = {static_cast<uint32_t>(va), static_cast<uint32_t>(va >> 32) & 0xFFFFu,
                          PV8 ? static_cast<uint32_t>(D) * p.np - n0 : static_cast<uint32_t>(min(N - n0, BN) * D * 2),
                          static_cast<uint32_t>(kBufferFlags)};
        const uint32_t stage = smem_lds + (t % C::STAGES) * C::STAGE;
        const int b0 = (grp == 0 ? 0 : DMA_A) + (w & 3);
#pragma unroll
        for (int i = 0; i < DMA_PER_W; ++i) {
            if (i < dma_n) {
                const int b = b0 + 4 * i;
                poison_block(stage + 1024 * b);
                lds_dma16(stage + 1024 * b, b < DMA_K ? kr : vr, dma_off[i]);
            }
        }
    };
    auto load_tile = [&](int t) {
        if constexpr (C::DMA) {
            dma_tile(t);
            if constexpr (PV8) {
                if (tid < C::SBYTES / 16)
                    sst = ld16(p.vscale + (static_cast<size_t>(bh) * n_all_tiles + tile_of(t)) * D + 16 * tid);
            }
            return;
        }
        const int n0 = tile_of(t) * BN;
        // (byte counts fit 32 bits: B*H*N*d < 2^31 elements of at most 2 bytes)
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(kg + static_cast<size_t>(n0) * D * ES), 0,
            static_cast<int>(static_cast<uint32_t>(min(N - n0, BN) * D * ES)), kBufferFlags);
        const __amdgpu_buffer_rsrc_t vr = PV8
            ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vg + n0), 0,
                                                static_cast<int>(static_cast<uint32_t>(D) * p.np - n0), kBufferFlags)
            : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vg + static_cast<size_t>(n0) * D * 2), 0,
                                                static_cast<int>(static_cast<uint32_t>(min(N - n0, BN) * D * 2)),
                                                kBufferFlags);
        if constexpr (PV8) {
            if (tid < C::SBYTES / 16)
                sst = ld16(p.vscale + (static_cast<size_t>(bh) * n_all_tiles + tile_of(t)) * D + 16 * tid);
        }
#pragma unroll
        for (int i = 0; i < C::K_PER_T; ++i) {
            const int c = i * NT + tid;
            if (c < C::K_CHUNKS) {
                const int row = c / C::K_CPR, col = c - row * C::K_CPR;
                kst[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, row * D * ES + 16 * col, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < C::V_PER_T; ++i) {
            const int c = i * NT + tid;
            if (c < C::V_CHUNKS) {
                const int row = c / C::V_CPR, col = c - row * C::V_CPR;   // key row (FP8 P*V: V^T row)
                vst[i] = __builtin_amdgcn_raw_buffer_load_b128(
                    vr, PV8 ? static_cast<int>(static_cast<uint32_t>(row) * p.np + 16 * col) : row * D * 2 + 16 * col,
                    0, 0);
            }
        }
    };
    auto store_tile = [&](int t) {
        if constexpr (C::DMA) {
            wait_lds_dma();
            if constexpr (PV8) {
                if (tid < C::SBYTES / 16)
                    *reinterpret_cast<u32x4*>(smem + (t % C::STAGES) * C::STAGE + C::KBYTES + C::VBYTES + 16 * tid) = sst;
            }
            return;
        }
        uint8_t* ks = smem + (t % C::STAGES) * C::STAGE;
        uint8_t* vs = ks + C::KBYTES;
#pragma unroll
        for (int i = 0; i < C::K_PER_T; ++i) {
            const int c = i * NT + tid;
            if (c < C::K_CHUNKS) {
                const int row = c / C::K_CPR, col = c - row * C::K_CPR;
                *reinterpret_cast<u32x4*>(ks + row * C::KROW + 16 * col) = kst[i];
            }
        }
#pragma unroll
        for (int i = 0; i < C::V_PER_T; ++i) {
            const int c = i * NT + tid;
            if (c < C::V_CHUNKS) {
                const int row = c / C::V_CPR, col = c - row * C::V_CPR;
                // v_granule is an involution in the granule index: data granule col
                // goes to LDS granule v_granule(row, col)
                const int pos = PV8 ? col : v_granule<D>(row, col);
                *reinterpret_cast<u32x4*>(vs + row * C::VROW + 16 * pos) = vst[i];
            }
        }
        if constexpr (PV8) {
            if (tid < C::SBYTES / 16) *reinterpret_cast<u32x4*>(vs + C::VBYTES + 16 * tid) = sst;
        }
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] = 0.0f;
    float m_run = kNegInf, l_run = 0.0f;
    float s[BN / 2];
    bf16x8 pf[BN / 16];
    uint32_t pf8[BN / 8] = {};                   // FP8 P*V: the lane's 32 P values as e4m3 codes
    int p_scale = 127;                           // FP8 P*V: block exponent of those codes

    // per-lane LDS addresses of this lane's K row / e4m3 V^T row fragments in stage 0
    const uint8_t* lane_k = smem + l32 * C::KROW + 16 * h;
    const uint8_t* lane_v = smem + C::KBYTES + l32 * C::VROW + 32 * h;
    // bf16 V: A operand of O^T += V^T P^T for 32 head dims (db) and 16 keys
    // (chunk cc).  The MFMA's k index 8h + t meets key 16cc + 4h + 8(t >> 2) +
    // (t & 3) in the probability fragment (the S^T accumulator layout), so lane
    // (dim 32db + l32, half h) needs V[16cc + 4h + {0..3}][dim] and
    // V[16cc + 8 + 4h + {0..3}][dim]: two transposing reads, in which lane
    // 16g + 4r + j names dims 32db + 16(g & 1) + 4j .. +3 of key row
    // 16cc + 4(g >> 1) + r (+ 8).  Byte offset of the first read of chunk 0,
    // within a stage's V tile, per db:
    uint32_t lane_vo[D / 32];
    {
        const int g = lane >> 4, r = (lane >> 2) & 3, j = lane & 3;
        const int t = D == 128 ? r : (D == 64 ? (r >> 1) & 1 : 0);    // the row's swizzle, in granule quads
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            lane_vo[db] = (4 * (g >> 1) + r) * C::VROW + 64 * (db ^ t) + 16 * (2 * (g & 1) + (j >> 1)) + 8 * (j & 1);
    }

    // ---- the four ops of the schedule
    // S^T = K_j Q^T for tile j
    auto op_s = [&](int j) {
        const uint8_t* ks = smem + (j % C::STAGES) * C::STAGE;
        if constexpr (!FP8) {
            // bf16: all K fragments first, MFMAs of the two 32-key blocks interleaved.
            // One per-lane address per tile; the fragments differ by immediate offsets.
            const uint8_t* kl = lane_k + (j % C::STAGES) * C::STAGE;
            constexpr int NA = (BN / 32) * C::QREGS;
            bf16x8 a[NA];
#pragma unroll
            for (int i = 0; i < C::QREGS; ++i)
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)
                    a[i * (BN / 32) + kb] = __builtin_bit_cast(bf16x8, ld16(kl + 32 * kb * C::KROW + 32 * i));
            f32x16 acc[BN / 32];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) acc[kb] = f32x16{};
#pragma unroll
            for (int i = 0; i < C::QREGS; ++i)
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)
                    acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i * (BN / 32) + kb],
                                                                     __builtin_bit_cast(bf16x8, qf[i]), acc[kb], 0, 0, 0);
            pipeline_lds_mfma<NA, kLdsAhead>();
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) s[16 * kb + v] = acc[kb][v];
            return;
        }
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 acc = {};
            const uint8_t* krow = ks + (32 * kb + l32) * C::KROW;
#pragma unroll
            for (int i = 0; i < C::QREGS; ++i) {
                if constexpr (C::F8W) {
                    const u32x4 a0 = ld16(krow + 64 * i + 32 * h);
                    const u32x4 a1 = ld16(krow + 64 * i + 32 * h + 16);
                    const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                     (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                    const u32x4 b0 = qf[2 * i], b1 = qf[2 * i + 1];
                    const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                                     (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
                    // fp8 e4m3 x fp8 e4m3, plain products: with both scale operands 0 the
                    // compiler emits the unscaled v_mfma_f32_32x32x64_f8f6f4 (no scale load)
                    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
                } else if constexpr (C::F8N) {
                    const long a = __builtin_bit_cast(long, *reinterpret_cast<const u32x2*>(krow + 16 * i + 8 * h));
                    const long b = __builtin_bit_cast(long, u32x2{qf[i][0], qf[i][1]});
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, acc, 0, 0, 0);
                } else {
                    const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(krow + 2 * (16 * i + 8 * h)));
                    const bf16x8 b = __builtin_bit_cast(bf16x8, qf[i]);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) s[16 * kb + v] = acc[v];
        }
    };
    // O^T += V_j^T P^T for tile j
    auto op_pv = [&](int j) {
        if constexpr (PV8) {
            const uint8_t* vl = lane_v + (j % C::STAGES) * C::STAGE;
            // O^T += V^T P^T on the 32x32x64 e4m3 MFMA: one per 32 rows of d covers the
            // whole 64-key tile; both operands carry their power-of-two block exponents
            const uint8_t* sc = smem + (j % C::STAGES) * C::STAGE + C::KBYTES + C::VBYTES;
            const i32x8 b = {(int)pf8[0], (int)pf8[1], (int)pf8[2], (int)pf8[3],
                             (int)pf8[4], (int)pf8[5], (int)pf8[6], (int)pf8[7]};
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const u32x4 a0 = ld16(vl + 32 * db * C::VROW);
                const u32x4 a1 = ld16(vl + 32 * db * C::VROW + 16);
                const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                 (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                const int sa = sc[32 * db + l32];
                o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, o[db], 0, 0, 0, sa, 0, p_scale);
            }
            return;
        }
        constexpr int NA = (D / 32) * (BN / 16);
        bf16x8 a[NA];
        const lds_u8* vs = (const lds_u8*)smem + (j % C::STAGES) * C::STAGE + C::KBYTES;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const lds_u8* vb = vs + lane_vo[db];
#pragma unroll
            for (int cc = 0; cc < BN / 16; ++cc) {
                const i16x4 lo = ds_read_tr16(vb + 16 * cc * C::VROW);
                const i16x4 hi = ds_read_tr16(vb + (16 * cc + 8) * C::VROW);
                a[db * (BN / 16) + cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int cc = 0; cc < BN / 16; ++cc)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[db * (BN / 16) + cc], pf[cc], o[db], 0, 0, 0);
        pipeline_lds_mfma<NA, kLdsAhead, 2>();
    };
    // softmax of tile j, rescale of O, probabilities packed to bf16
    auto op_softmax = [&](int j, bool masked) {
        const int n0 = tile_of(j) * BN;
        if (masked) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = n0 + 32 * kb + acc_row(v, h);
                    if (key >= N || (CAUSAL && key > my_q)) s[16 * kb + v] = kNegInf;
                }
        }
        float c = c_q;
        // BN = 64: tile j is scale tile j (a scalar load and a reciprocal, as in the
        // 128-key kernel)
        if (FP8) c = c_q * __builtin_amdgcn_rcpf(((const const_f32*)(p.k_scale))[bh * n_scale + tile_of(j)]);
        float alpha;
        if constexpr (PV8) alpha = softmax_step_p8(s, c, m_run, l_run, p_scale);
        else alpha = softmax_step(s, c, m_run, l_run);
        // with the lazy reference max, alpha is 1 for every lane on most tiles:
        // skip the 16*D/32 multiplies then (a wave-uniform branch)
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
        }
        if constexpr (PV8) {
            // byte t of the B operand is s[t] (register order = the k-slot order of f8_slot);
            // the two packs overwrite both halves of the previous tile's word, which is
            // passed as the preserved half so that no zero has to be written first
#pragma unroll
            for (int wd = 0; wd < BN / 8; ++wd) {
                int x = __builtin_amdgcn_cvt_pk_fp8_f32(s[4 * wd], s[4 * wd + 1], static_cast<int>(pf8[wd]), false);
                x = __builtin_amdgcn_cvt_pk_fp8_f32(s[4 * wd + 2], s[4 * wd + 3], x, true);
                pf8[wd] = static_cast<uint32_t>(x);
            }
        } else {
#pragma unroll
            for (int cc = 0; cc < BN / 16; ++cc)
#pragma unroll
                for (int t = 0; t < 8; ++t) pf[cc][t] = static_cast<__bf16>(s[8 * cc + t]);
        }
    };
    // this wave's share of the tile traffic in V_j: publish tile j+lead, prefetch tile j+lead+1
    const int lead = grp == 0 ? 1 : 2;
    auto traffic = [&](int j) {
        const int ts = j + lead;
        if (ts < n_kt) store_tile(ts);
        if (ts + 1 < n_kt) load_tile(ts + 1);
    };

    // ---- prologue: group A publishes its half of tile 0, group B of tiles 0 and 1
    for (int t = 0; t < lead && t < n_kt; ++t) {
        load_tile(t);
        store_tile(t);
    }
    if (lead < n_kt) load_tile(lead);
    lds_barrier();
    if (grp == 1) lds_barrier();                  // group B idles through slot 0

    // ---- slots.  Barrier k (k = 1, 2, ...) of this wave ends its op k-1:
    //      M_0 | V_0 M_1 | V_1 M_2 | ... | V_{n-1} M_n
    // Tiles before j_last need no mask (their last key precedes this wave's
    // first query, and only the last tile can hold keys >= N).
    if (SPARSE) {
        // the same slots over the listed tiles; a wave skips the work of a tile
        // its 64-query block does not need (or that lies above its diagonal)
        if (needs(0)) op_s(0);
        lds_barrier();
        for (int j = 0; j < n_kt; ++j) {
            const bool nj = needs(j);
            const int n0 = tile_of(j) * BN;
            if (nj) op_softmax(j, (CAUSAL && n0 + BN - 1 > qw0) || n0 + BN > N);
            traffic(j);
            lds_barrier();
            if (nj) op_pv(j);
            __builtin_amdgcn_sched_barrier(0);
            if (j + 1 < n_kt && needs(j + 1)) op_s(j + 1);
            lds_barrier();
        }
    } else if (PARTIAL && j_last < 0) {
        // every key of the range comes after this wave's queries: it only
        // publishes its share of the tiles, in the same slots as the others
        lds_barrier();
        for (int j = 0; j < n_kt; ++j) {
            traffic(j);
            lds_barrier();
            lds_barrier();
        }
    } else {
        op_s(0);
        lds_barrier();
        for (int j = 0; j < j_last; ++j) {
            op_softmax(j, false);
            traffic(j);
            lds_barrier();
            op_pv(j);
            __builtin_amdgcn_sched_barrier(0);
            op_s(j + 1);
            lds_barrier();
        }
        {
            const int n0 = (lo + j_last) * BN;
            op_softmax(j_last, (CAUSAL && n0 + BN - 1 > qw0) || n0 + BN > N);
            traffic(j_last);
            lds_barrier();
            op_pv(j_last);
            lds_barrier();
        }
        for (int j = j_last + 1; j < n_kt; ++j) { // this wave is past the diagonal: traffic only
            traffic(j);
            lds_barrier();
            lds_barrier();
        }
    }
    if (grp == 0) lds_barrier();                  // group A idles through the last slot
    if constexpr (C::DMA) wait_lds_dma();         // no copy may land after the workgroup ends

    // ---- epilogue
    const float l_tot = sum_halves(l_run);
    if (PARTIAL) {
        // O normalised over this split's keys, in fp32, and the split's lse (-inf if it saw no key)
        if (my_q < N) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            const size_t row = (static_cast<size_t>(split) * p.BH + bh) * N + my_q;
            float* orow = p.o32 + row * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = o[db][4 * g + e] * inv;
                    *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * h) = out;
                }
            if (h == 0) p.lse_part[row] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
        }
        return;
    }
    if (my_q < N) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint8_t* orow = p.o + (slice + static_cast<size_t>(my_q) * D) * 2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(o[db][4 * g + e] * inv);
                *reinterpret_cast<bf16x4*>(orow + 2 * (32 * db + 8 * g + 4 * h)) = out;
            }
        if (p.lse != nullptr && h == 0)
            p.lse[static_cast<size_t>(bh) * N + my_q] = (m_run + __log2f(l_tot)) * kLn2;
    }
}

// ===========================================================================
// bf16, d = 128: the same ping-pong schedule with 128 keys per slot
//
// Each matrix-core slot covers 128 keys (64 MFMAs per wave instead of 32), so
// the fixed cost of a slot -- the wait for the first LDS operands, the
// barrier -- is paid once per 128 keys.  K and V tiles live in two separate
// double-buffered rings (K 128 x 272 B, V 128 x 256 B per stage: 132 KiB):
// K_t is read by S_t in slots 2t (group A) and 2t+1 (group B), V_t by PV_t in
// slots 2t+2 and 2t+3.  Group B copies both, in its vector slot 2j+2: K_{j+2}
// into the stage K_j left (last read in slot 2j+1) and V_{j+1} into the stage
// V_{j-1} left (last read in slot 2j+1); it waits for them at the end of slot
// 2j+3, before the barrier after which group A first reads them.  Copies are
// LDS-DMA blocks of 1 KiB as in the 64-key kernel.
// ===========================================================================
// s_waitcnt vmcnt(N): all but this wave's last N vector-memory loads (here
// LDS-DMA copies, which complete in issue order) have landed
template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

template <bool FP8, bool PV8 = false>
struct B128Cfg {
    static constexpr int D = 128, NW = 8, NT = 64 * NW, BM = 32 * NW, BN = 128;
    static constexpr int ES = FP8 ? 1 : 2;     // bytes per Q/K element (e4m3 or bf16)
    // V: BN natural bf16 key rows; e4m3 P*V: D rows of V^T, BN keys plus one pad granule
    static constexpr int KROW = D * ES + 16, VROW = PV8 ? BN + 16 : D * 2;
    // a K stage holds BN padded rows (34 KiB, e4m3 18 KiB); it is rounded up to
    // whole groups of four blocks so that each of the four copying waves issues
    // the same number (the last blocks carry no data).  An e4m3 V^T stage is
    // 18 KiB of rows, then one block whose first 2 x D bytes are the block
    // exponents of the tile's two 64-key halves, rounded up the same way.
    static constexpr int K_BLOCKS = (BN * KROW + 4095) / 4096 * 4;
    static constexpr int V_DATA = (PV8 ? D : BN) * VROW / 1024;
    static constexpr int V_BLOCKS = PV8 ? (V_DATA + 1 + 3) / 4 * 4 : V_DATA;
    static constexpr int VSCALE = V_DATA * 1024;    // e4m3 P*V: byte offset of the exponents in a V stage
    static constexpr int KSTAGE = K_BLOCKS * 1024, VSTAGE = V_BLOCKS * 1024;
    static constexpr int K_PER_W = K_BLOCKS / 4, V_PER_W = V_BLOCKS / 4;
    // Q fragments per lane: 16 dims per bf16 MFMA; e4m3: 64 dims per MFMA, 32 bytes a lane
    static constexpr int QREGS = FP8 ? 2 * (D / 64) : D / 16;
    // K stages: FP8 keeps three (see the copy schedule in the kernel), bf16 two
    static constexpr int KST = FP8 ? 3 : 2;
    static constexpr int SMEM = KST * KSTAGE + 2 * VSTAGE;
    static constexpr int AHEAD = 9;            // LDS operand lookahead, in MFMAs (9 measured 0.7 % faster than 6)
};

template <bool CAUSAL, bool FP8, bool PV8 = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_b128_kernel(KParams p) {
    using C = B128Cfg<FP8, PV8>;
    constexpr int D = C::D, BM = C::BM, BN = C::BN, ES = C::ES;
    static_assert(C::KSTAGE % 1024 == 0 && C::VSTAGE % 4096 == 0, "LDS-DMA layout");
    static_assert(!PV8 || (FP8 && C::D * C::VROW == C::V_DATA * 1024), "e4m3 P*V: e4m3 S, whole V^T blocks");
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::SMEM];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, grp = w >> 2, h = lane >> 5, l32 = lane & 31;
    const int N = p.N;
    // Work item.  Query-tile major (band = 0): workgroup b takes head b mod BH.
    // XCD-banded (band > 0, BH a multiple of 8): XCD x = b mod 8 runs heads
    // x + 8m; its k-th workgroup (k = b / 8) is in band k / (band n_qtiles),
    // which holds `band` of those heads, walked query tile by query tile
    // (heaviest first when causal) across the band's heads.  The query tiles
    // of a band stream the same few heads' K and V at about the same time, so
    // the XCD's L2 serves most of their reads.
    int qt, bh;
    if (p.band > 0) {
        const int x = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
        const int per_band = p.band * p.n_qtiles;
        const int band = k / per_band, r = k - band * per_band;
        qt = r / p.band;
        bh = x + kXcds * (band * p.band + (r - qt * p.band));
    } else {
        qt = blockIdx.x / p.BH;
        bh = blockIdx.x - qt * p.BH;
    }
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;        // heaviest query tiles first
    const int q0 = qt * BM, qw0 = q0 + 32 * w, my_q = qw0 + l32;
    const size_t slice = static_cast<size_t>(bh) * N * D;
    const uint8_t* qg = p.q + slice * ES;
    const uint8_t* kg = p.k + slice * ES;
    // V rows of this (b, h), or (e4m3 P*V) its e4m3 V^T: D rows of np keys
    const uint8_t* vg = PV8 ? p.vt + static_cast<size_t>(bh) * D * p.np : p.v + slice * 2;

    // Q fragments (B operand): bf16 dims 16i + 8h .. +7; e4m3 dims 64(i/2) + 32h + 16(i%2) .. +15
    u32x4 qf[C::QREGS];
    {
        const bool ok = my_q < N;
        const uint8_t* row = qg + static_cast<size_t>(my_q) * D * ES;
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i)
            qf[i] = !ok ? u32x4{0, 0, 0, 0} : FP8 ? ld16(row + 64 * (i >> 1) + 32 * h + 16 * (i & 1)) : ld16(row + 2 * (16 * i + 8 * h));
    }
    // scores in base-2 units: s * c (FP8: with the dequantisation 1/(q_scale k_scale),
    // the K scale per 64-key half of a tile)
    const int n_scale = (N + 63) / 64;
    float c_q = p.c_log2;
    if constexpr (FP8) c_q = p.c_log2 / p.q_scale[bh * n_scale + (qw0 < N ? qw0 : N - 1) / 64];

    const int n_all = (N + BN - 1) / BN;
    const int n_kt = CAUSAL ? min(n_all, (min(q0 + BM, N) + BN - 1) / BN) : n_all;
    // last key tile with a key at or before this wave's last query
    const int j_last = CAUSAL ? min(n_kt - 1, (qw0 + 31) / BN) : n_kt - 1;

    // ---- tile copies (group B): per-lane source offsets of its K blocks (padded
    // rows: 16 granules + one pad granule) and of its first V block (V blocks
    // of one wave are 16 key rows = 4 KiB of source apart)
    const uint32_t smem_lds = lds_address(smem);
    const uint32_t kbase = smem_lds, vbase = smem_lds + C::KST * C::KSTAGE;
    uint32_t k_off[C::K_PER_W];
    uint32_t v_off0 = 0;
    // e4m3 V^T: per-lane offsets of this wave's V blocks (rows of np keys: D rows of
    // 8 granules + one pad granule, then the exponent block: 16 lanes of 16 bytes)
    uint32_t v_off8[PV8 ? C::V_PER_W : 1];
    {
#pragma unroll
        for (int i = 0; i < C::K_PER_W; ++i)
            k_off[i] = dma_lane_offset((w & 3) + 4 * i, lane, D * ES / 16, D * ES, BN);   // past row BN: no data
        const int row = 4 * (w & 3) + (lane >> 4);
        v_off0 = row * (D * 2) + 16 * v_granule<D>(row, lane & 15);
        if constexpr (PV8) {
#pragma unroll
            for (int i = 0; i < C::V_PER_W; ++i) {
                const int b = (w & 3) + 4 * i, g = 64 * b + lane, vr = g / (BN / 16 + 1), col = g - (BN / 16 + 1) * vr;
                v_off8[i] = b < C::V_DATA ? (col < BN / 16 ? static_cast<uint32_t>(vr) * p.np + 16 * col : 0x40000000u)
                                          : (b == C::V_DATA && lane < 2 * D / 16 ? 16u * lane : 0x40000000u);
            }
        }
    }
    // block (w & 3) + 4i of a stage: LDS byte 1024 (w & 3) + 4096 i of it
    auto copy_k = [&](int t) {                    // K_t into K stage t % 2
        const int n0 = t * BN;
        const u32x4 r = buffer_words(kg + static_cast<size_t>(n0) * D * ES, static_cast<uint32_t>(min(N - n0, BN) * D * ES));
        const uint32_t st = kbase + (t % C::KST) * C::KSTAGE + 1024 * (w & 3);
        static_for<0, C::K_PER_W>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            poison_block(st + 4096 * i);
            lds_dma16_at<4096 * i, 0>(st, r, k_off[i]);
        });
    };
    auto copy_v = [&](int t) {                    // V_t into V stage t % 2; its rows 16 i further on
        const int n0 = t * BN;
        const uint32_t st = vbase + (t & 1) * C::VSTAGE + 1024 * (w & 3);
        if constexpr (PV8) {
            // e4m3 V^T columns n0 .. n0 + BN (past np: zero or the next row's codes,
            // met by P = 0) and the exponents of 64-key tiles 2t, 2t + 1 (past the
            // last: 0, a finite 2^-127)
            const int n64 = (N + 63) / 64;
            const u32x4 r = buffer_words(vg + n0, static_cast<uint32_t>(D) * p.np - n0);
            const u32x4 rs = buffer_words(p.vscale + (static_cast<size_t>(bh) * n64 + 2 * t) * D,
                                          static_cast<uint32_t>(min(2, n64 - 2 * t) * D));
            // blocks of the last round: data for waves with (w & 3) + 4 i < V_DATA, the
            // exponents for the next one, nothing (offset past every range) after it
            static_assert(C::V_DATA >= 4 * (C::V_PER_W - 1) && C::V_DATA < 4 * C::V_PER_W, "one mixed round");
            const bool last_data = (w & 3) < C::V_DATA - 4 * (C::V_PER_W - 1);
            const u32x4 rl = {last_data ? r[0] : rs[0], last_data ? r[1] : rs[1], last_data ? r[2] : rs[2],
                              last_data ? r[3] : rs[3]};
            static_for<0, C::V_PER_W>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                poison_block(st + 4096 * i);
                lds_dma16_at<4096 * i, 0>(st, i + 1 < C::V_PER_W ? r : rl, v_off8[i]);
            });
            return;
        }
        const u32x4 r = buffer_words(vg + static_cast<size_t>(n0) * D * 2, static_cast<uint32_t>(min(N - n0, BN) * D * 2));
        static_for<0, C::V_PER_W>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            poison_block(st + 4096 * i);
            lds_dma16_at<4096 * i, 16 * i * C::VROW>(st, r, v_off0);
        });
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] = 0.0f;
    float m_run = kNegInf, l_run = 0.0f;
    float s[BN / 2];
    bf16x8 pf[BN / 16];
    uint32_t pf8[2][8] = {};                      // e4m3 P*V: P^T of each 64-key half, e4m3 codes
    int p_scale[2] = {127, 127};                  // and their block exponents (127 - f)

    const uint8_t* lane_k = smem + l32 * C::KROW + 16 * h;
    uint32_t lane_vo[D / 32];
    {
        const int g = lane >> 4, r = (lane >> 2) & 3, j = lane & 3;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            lane_vo[db] = (4 * (g >> 1) + r) * C::VROW + 64 * (db ^ r) + 16 * (2 * (g & 1) + (j >> 1)) + 8 * (j & 1);
    }

    // S^T = K_t Q^T over the 128 keys of tile t
    auto op_s = [&](int t) {
        const uint8_t* kl = lane_k + (t % C::KST) * C::KSTAGE;
        if constexpr (FP8) {
            // e4m3: one 32x32x64 MFMA per 32 keys and 64 dims; a lane's 32 bytes of a K row
            // (dims 64i + 32h ..) are two 16-byte reads
            constexpr int NI = D / 64, NA = (BN / 32) * NI;
            i32x8 a[NA];
            const uint8_t* kf = smem + (t % C::KST) * C::KSTAGE + l32 * C::KROW + 32 * h;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb) {
                    const u32x4 a0 = ld16(kf + 32 * kb * C::KROW + 64 * i);
                    const u32x4 a1 = ld16(kf + 32 * kb * C::KROW + 64 * i + 16);
                    a[i * (BN / 32) + kb] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                                  (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                }
            f32x16 acc[BN / 32];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) acc[kb] = f32x16{};
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const u32x4 b0 = qf[2 * i], b1 = qf[2 * i + 1];
                const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)   // e4m3 x e4m3, plain products (scale operands 0:
                                                        // the unscaled v_mfma_f32_32x32x64_f8f6f4)
                    acc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i * (BN / 32) + kb], b, acc[kb], 0, 0, 0,
                                                                              0, 0, 0);
            }
            pipeline_lds_mfma<NA, C::AHEAD / 2, 2>();
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) s[16 * kb + v] = acc[kb][v];
            return;
        }
        constexpr int NA = (BN / 32) * C::QREGS;
        bf16x8 a[NA];
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i)
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
                a[i * (BN / 32) + kb] = __builtin_bit_cast(bf16x8, ld16(kl + 32 * kb * C::KROW + 32 * i));
        f32x16 acc[BN / 32];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) acc[kb] = f32x16{};
#pragma unroll
        for (int i = 0; i < C::QREGS; ++i)
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
                acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i * (BN / 32) + kb], __builtin_bit_cast(bf16x8, qf[i]),
                                                                 acc[kb], 0, 0, 0);
        pipeline_lds_mfma<NA, C::AHEAD>();
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[16 * kb + v] = acc[kb][v];
    };
    // O^T += V_t^T P_t^T
    auto op_pv = [&](int t) {
        if constexpr (PV8) {
            // one 32x32x64 e4m3 MFMA per 64-key half and 32 rows of d; A = 32 bytes of a
            // V^T row (keys 32h .. of the half, in the P operand's key order), both
            // operands scaled by their block exponents
            const uint8_t* vl = smem + C::KST * C::KSTAGE + (t & 1) * C::VSTAGE;
            const uint8_t* sc = vl + C::VSCALE;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const i32x8 b = {(int)pf8[hf][0], (int)pf8[hf][1], (int)pf8[hf][2], (int)pf8[hf][3],
                                 (int)pf8[hf][4], (int)pf8[hf][5], (int)pf8[hf][6], (int)pf8[hf][7]};
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const uint8_t* ap = vl + (32 * db + l32) * C::VROW + 64 * hf + 32 * h;
                    const u32x4 a0 = ld16(ap), a1 = ld16(ap + 16);
                    const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                     (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                    const int sa = sc[D * hf + 32 * db + l32];
                    o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, o[db], 0, 0, 0, sa, 0, p_scale[hf]);
                }
            }
            pipeline_lds_mfma<2 * (D / 32), 3, 3>();    // two operand reads and the exponent byte per MFMA
            return;
        }
        constexpr int NA = (D / 32) * (BN / 16);
        bf16x8 a[NA];
        const lds_u8* vs = (const lds_u8*)smem + C::KST * C::KSTAGE + (t & 1) * C::VSTAGE;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const lds_u8* vb = vs + lane_vo[db];
#pragma unroll
            for (int cc = 0; cc < BN / 16; ++cc) {
                const i16x4 lo = ds_read_tr16(vb + 16 * cc * C::VROW);
                const i16x4 hi = ds_read_tr16(vb + (16 * cc + 8) * C::VROW);
                a[db * (BN / 16) + cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int cc = 0; cc < BN / 16; ++cc)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[db * (BN / 16) + cc], pf[cc], o[db], 0, 0, 0);
        pipeline_lds_mfma<NA, C::AHEAD, 2>();
    };
    // softmax of tile t, rescale of O, probabilities packed to bf16
    auto op_softmax = [&](int t, bool masked) {
        if (masked) {
            // key t*BN + 4h + c is visible iff c <= lim
            const int lim = (CAUSAL ? min(N - 1, my_q) : N - 1) - t * BN - 4 * h;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (32 * kb + 8 * (v >> 2) + (v & 3) > lim) s[16 * kb + v] = kNegInf;   // acc_row(v, h) - 4h
        }
        float c0 = c_q, c1 = c_q;
        if constexpr (FP8) {
            // 64-key halves carry their own K scales (64-row scale tiles); the second
            // half of the last tile may lie past N (then its scale is never used)
            // (scalar loads: a vector load's wait would also wait for this wave's
            // tile copies in flight; a reciprocal instead of an IEEE division, within
            // an ulp or two)
            const int ks = bh * n_scale + 2 * t;
            const const_f32* kscale = (const const_f32*)(p.k_scale);
            c0 = c_q * __builtin_amdgcn_rcpf(kscale[ks]);
            c1 = 2 * t + 1 < n_scale ? c_q * __builtin_amdgcn_rcpf(kscale[ks + 1]) : c0;
        }
        if constexpr (PV8) {
            // the scale of each half's probabilities needs that half's max: always the full step
            const float alpha = softmax_step_p8x2(s, c0, c1, m_run, l_run, p_scale);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
            }
            // byte 4 wd + k of half hf's B operand is s[32 hf + 4 wd + k] (register order =
            // the key order of the e4m3 V^T rows)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int wd = 0; wd < 8; ++wd) {
                    int x = __builtin_amdgcn_cvt_pk_fp8_f32(s[32 * hf + 4 * wd], s[32 * hf + 4 * wd + 1],
                                                            static_cast<int>(pf8[hf][wd]), false);   // both halves rewritten
                    x = __builtin_amdgcn_cvt_pk_fp8_f32(s[32 * hf + 4 * wd + 2], s[32 * hf + 4 * wd + 3], x, true);
                    pf8[hf][wd] = static_cast<uint32_t>(x);
                }
            return;
        }
        // FP8: past the first tile, the probabilities against the current reference
        // first (softmax_at_ref), the full step only where that fails.  (Measured:
        // FP8 +1-2 %; bf16 -0.3 % at 1x32x16384x128 causal, -1 % at 4x32x4096x128,
        // so bf16 always takes the full step.)
        if (!FP8 || t == 0 || !softmax_at_ref(s, c0, c1, m_run, l_run, pf)) {
            const float alpha = FP8 ? softmax_step2(s, c0, c1, m_run, l_run) : softmax_step(s, c_q, m_run, l_run);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
            }
#pragma unroll
            for (int cc = 0; cc < BN / 16; ++cc)
#pragma unroll
                for (int t8 = 0; t8 < 8; ++t8) pf[cc][t8] = static_cast<__bf16>(s[8 * cc + t8]);
        }
    };
    auto masked_tile = [&](int t) { return (CAUSAL && t * BN + BN - 1 > qw0) || t * BN + BN > N; };
    // slot boundary: neither matrix-core nor vector work crosses it (left to
    // itself the scheduler moves MFMAs into the vector slot and exps into the
    // matrix slot, which measured slower)
    auto slot_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: group B copies K_0 and waits; everyone meets at barrier 0
    if (grp == 1) {
        copy_k(0);
        wait_lds_dma();
    }
    lds_barrier();

    // Tiles before j_last need no mask (their last key precedes this wave's first
    // query, and only the last tile can hold keys >= N); the masked tile j_last
    // is peeled off the loops so that the masking code stays out of them.
    const bool last_masked = masked_tile(j_last);
    // Who copies.  bf16: group B copies K_{j+2} and V_{j+1} in slot 2j+2, after
    // its softmax, and waits for them at the end of slot 2j+3.  FP8 (e4m3 S, so
    // the matrix-core slot is ~1 000 cycles shorter than the vector slot): group A
    // copies, K_{j+2} at the start of its vector slot 2j+1 (into the third K
    // stage, which K_{j-1} left in slot 2j-1) and V_{j+1} after its MFMAs in slot
    // 2j+2; at the end of slot 2j+1 it waits for all but the K copies just issued.
    // Issued in one burst, the copies queue behind the CU's address unit; this
    // puts that time where the schedule has slack.
    constexpr bool A_COPIES = FP8;
    auto copies = [&](int j) {
        if (j + 2 < n_kt) copy_k(j + 2);
        if (j + 1 < n_kt) copy_v(j + 1);
    };
    // A, end of vector slot 2j+1: K_{j+1} and V_j must have landed, K_{j+2} may not
    auto wait_a = [&](int j) {
        if (j + 2 < n_kt) wait_vmcnt<C::K_PER_W>();
        else wait_lds_dma();
    };
    if (grp == 0) {
        // A: M_0 | V_0 M_1 | ... | V_{n-1} M_n | idle
        op_s(0);
        slot_end();
        for (int j = 0; j < j_last; ++j) {
            if (A_COPIES && j + 2 < n_kt) copy_k(j + 2);
            op_softmax(j, false);
            if (A_COPIES) wait_a(j);
            slot_end();
            op_pv(j);
            __builtin_amdgcn_sched_barrier(0);
            op_s(j + 1);
            if (A_COPIES && j + 1 < n_kt) copy_v(j + 1);
            slot_end();
        }
        if (A_COPIES && j_last + 2 < n_kt) copy_k(j_last + 2);
        op_softmax(j_last, last_masked);
        if (A_COPIES) wait_a(j_last);
        slot_end();
        op_pv(j_last);
        if (A_COPIES && j_last + 1 < n_kt) copy_v(j_last + 1);
        slot_end();
        for (int j = j_last + 1; j < n_kt; ++j) {     // past the diagonal: slots (and copies) only
            if (A_COPIES && j + 2 < n_kt) copy_k(j + 2);
            if (A_COPIES) wait_a(j);
            slot_end();
            if (A_COPIES && j + 1 < n_kt) copy_v(j + 1);
            slot_end();
        }
        if (A_COPIES) wait_lds_dma();
        slot_end();
    } else {
        // B: copies | M_0 | V_0 (+ copies), M_1 | ... | V_{n-1} (+ copies), M_n
        if (1 < n_kt) copy_k(1);
        copy_v(0);
        slot_end();
        op_s(0);
        wait_lds_dma();
        slot_end();
        for (int j = 0; j < j_last; ++j) {
            op_softmax(j, false);
            if (!A_COPIES) copies(j);
            slot_end();
            op_pv(j);
            __builtin_amdgcn_sched_barrier(0);
            op_s(j + 1);
            if (!A_COPIES) wait_lds_dma();
            slot_end();
        }
        op_softmax(j_last, last_masked);
        if (!A_COPIES) copies(j_last);
        slot_end();
        op_pv(j_last);
        if (!A_COPIES) wait_lds_dma();
        slot_end();
        for (int j = j_last + 1; j < n_kt; ++j) {     // past the diagonal: copies for the others
            if (!A_COPIES) copies(j);
            slot_end();
            if (!A_COPIES) wait_lds_dma();
            slot_end();
        }
    }

    // ---- epilogue
    const float l_tot = sum_halves(l_run);
    if (my_q < N) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint8_t* orow = p.o + (slice + static_cast<size_t>(my_q) * D) * 2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(o[db][4 * g + e] * inv);
                *reinterpret_cast<bf16x4*>(orow + 2 * (32 * db + 8 * g + 4 * h)) = out;
            }
        if (p.lse != nullptr && h == 0)
            p.lse[static_cast<size_t>(bh) * N + my_q] = (m_run + __log2f(l_tot)) * kLn2;
    }
}

// ===========================================================================
// bf16, d = 32: every wave runs its own tiles, one barrier per 256 keys
//
// At d = 32 a 64-key tile is 8 MFMAs per wave against ~120 vector
// instructions of softmax, so the vector ALUs bound the kernel, and a
// ping-pong split (one group on the matrix cores while the other runs the
// softmax, a barrier every 64 keys) leaves the copies too little time to land
// and pays its barriers on short slots.  Here each wave computes S, the
// softmax and P*V of a tile back to back, and the four waves a SIMD holds
// (two workgroups per CU) overlap one another's matrix and vector work on
// their own.  K and V arrive in stages of SK keys through a two-stage LDS-DMA
// ring: at the one barrier per stage the next stage's copy is issued into the
// buffer the last stage left, a whole stage of compute ahead of its use.
//
// Causal: workgroup i of a head takes the 128-query chunks i (waves 0-3) and
// NC - 1 - i (waves 4-7) of its NC chunks, so every workgroup has the same
// work, and so has every SIMD (one wave of each chunk).
// ===========================================================================
template <int SK_>
struct D32Cfg {
    static constexpr int D = 32, NW = 8, NT = 64 * NW, BM = 32 * NW, BN = 64;
    static constexpr int SK = SK_;               // keys per stage
    static constexpr int TPS = SK / BN;          // 64-key tiles per stage
    static constexpr int KROW = D * 2 + 16;      // K row in LDS: 4 granules + 1 pad granule
    static constexpr int VROW = D * 2;           // V row in LDS: natural, unpadded
    static constexpr int KBYTES = SK * KROW, VBYTES = SK * VROW;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int K_BLOCKS = KBYTES / 1024, BLOCKS = STAGE / 1024;
    static constexpr int PER_W = (BLOCKS + NW - 1) / NW;
    static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "LDS-DMA layout");
};

template <bool CAUSAL, int SK = 256, bool FAST = true>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
void fwd_d32_kernel(KParams p) {
    using C = D32Cfg<SK>;
    constexpr int D = C::D, BN = C::BN, TPS = C::TPS;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int N = p.N;
    const int wi = blockIdx.x / p.BH;           // workgroup of the head
    const int bh = blockIdx.x - wi * p.BH;
    // this wave's 32 query rows start at qw0; the workgroup needs keys [0, kend)
    int qw0, kend;
    bool rows = true;
    if (CAUSAL) {
        const int nc = (N + 127) / 128, c_hi = nc - 1 - wi;
        qw0 = 128 * (w < 4 ? wi : c_hi) + 32 * (w & 3);
        rows = w < 4 || c_hi != wi;             // odd NC: the middle chunk has one set of waves
        kend = min(N, 128 * c_hi + 128);
    } else {
        qw0 = C::BM * wi + 32 * w;
        kend = N;
    }
    rows = rows && qw0 < N;
    const int my_q = qw0 + l32;
    const size_t slice = static_cast<size_t>(bh) * N * D;
    const uint8_t* qg = p.q + slice * 2;
    const uint8_t* kg = p.k + slice * 2;
    const uint8_t* vg = p.v + slice * 2;

    const int n_st = (kend + SK - 1) / SK;
    // tiles of this wave: keys [0, min(N, qw0 + 32)) when causal; a wave without
    // rows only copies
    const int n_t = !rows ? 0 : ((CAUSAL ? min(N, qw0 + 32) : N) + BN - 1) / BN;

    // ---- stage copies: 1 KiB block b of a stage by wave b mod 8; K blocks hold
    // padded rows (dma_lane_offset), V blocks the tile's bytes in order
    const uint32_t smem_lds = lds_address(smem);
    uint32_t off[C::PER_W];
#pragma unroll
    for (int i = 0; i < C::PER_W; ++i) {
        const int b = w + C::NW * i;
        off[i] = b < C::K_BLOCKS ? dma_lane_offset(b, lane, D * 2 / 16, D * 2, SK)
                                 : static_cast<uint32_t>(1024 * (b - C::K_BLOCKS) + 16 * lane);
    }
    auto copy_stage = [&](int st) {
        const int n0 = st * SK;
        const uint32_t bytes = static_cast<uint32_t>(min(N - n0, SK) * D * 2);
        const u32x4 kr = buffer_words(kg + static_cast<size_t>(n0) * D * 2, bytes);
        const u32x4 vr = buffer_words(vg + static_cast<size_t>(n0) * D * 2, bytes);
        const uint32_t base = smem_lds + (st & 1) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::PER_W; ++i) {
            const int b = w + C::NW * i;
            if (b < C::BLOCKS) {
                poison_block(base + 1024 * b);
                lds_dma16(base + 1024 * b, b < C::K_BLOCKS ? kr : vr, off[i]);
            }
        }
    };

    f32x16 o = {};
    float m_run = kNegInf, l_run = 0.0f;
    float s[BN / 2];
    bf16x8 pf[BN / 16];
    u32x4 qf[2];

    // V^T operand of O^T += V^T P^T: lane 16g + 4r + j reads dims 16(g & 1) + 4j ..
    // of key row 16cc + 4(g >> 1) + r (+ 8) with the transposing read
    uint32_t lane_vo;
    {
        const int g = lane >> 4, r = (lane >> 2) & 3, j = lane & 3;
        lane_vo = (4 * (g >> 1) + r) * C::VROW + 16 * (2 * (g & 1) + (j >> 1)) + 8 * (j & 1);
    }

    // S^T = K Q^T for the tile at K row `kr0` of the stage whose lane address is kl
    auto op_s = [&](const uint8_t* kl) {
        bf16x8 a[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) a[2 * i + kb] = __builtin_bit_cast(bf16x8, ld16(kl + 32 * kb * C::KROW + 32 * i));
        f32x16 acc[2] = {};
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2 * i + kb], __builtin_bit_cast(bf16x8, qf[i]), acc[kb],
                                                                 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[16 * kb + v] = acc[kb][v];
    };
    bf16x8 va[4];                                 // V^T operand of the tile in flight
    auto read_v = [&](const lds_u8* vb) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const i16x4 lo = ds_read_tr16(vb + 16 * cc * C::VROW);
            const i16x4 hi = ds_read_tr16(vb + (16 * cc + 8) * C::VROW);
            va[cc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    auto op_pv = [&]() {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[cc], pf[cc], o, 0, 0, 0);
    };
    auto op_softmax = [&](int t) {
        const int n0 = t * BN;
        if ((CAUSAL && n0 + BN - 1 > qw0) || n0 + BN > N) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = n0 + 32 * kb + acc_row(v, h);
                    if (key >= N || (CAUSAL && key > my_q)) s[16 * kb + v] = kNegInf;
                }
        }
        if (FAST && t != 0 && softmax_at_ref(s, p.c_log2, p.c_log2, m_run, l_run, pf)) return;
        const float alpha = softmax_step(s, p.c_log2, m_run, l_run);
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) o[v] *= alpha;
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int t8 = 0; t8 < 8; ++t8) pf[cc][t8] = static_cast<__bf16>(s[8 * cc + t8]);
    };

    copy_stage(0);
    // Q fragments (B operand of S^T = K Q^T): dims 16i + 8h .. +7, loaded while
    // the first stage is on its way and waited for here: a wait left to the loop
    // (the compiler's vmcnt(0)) would also wait for the next stage's copies
    {
        const bool ok = my_q < N;
        const uint8_t* row = qg + static_cast<size_t>(my_q) * D * 2;
#pragma unroll
        for (int i = 0; i < 2; ++i) qf[i] = ok ? ld16(row + 2 * (16 * i + 8 * h)) : u32x4{0, 0, 0, 0};
        asm volatile("" : : "v"(qf[0]), "v"(qf[1]));
    }
    const uint8_t* lane_k = smem + l32 * C::KROW + 16 * h;
    const lds_u8* lane_v = (const lds_u8*)smem + C::KBYTES + lane_vo;
    for (int st = 0; st < n_st; ++st) {
        wait_lds_dma();                           // this wave's copies of stage st have landed
        lds_barrier();                            // so have everyone's; stage st - 1 is read
        if (st + 1 < n_st) copy_stage(st + 1);    // into the buffer stage st - 1 leaves
        // per tile: the V reads go out before the softmax and the next tile's S
        // after it, so that LDS and matrix-core latencies overlap this wave's
        // own vector work
        const int t0 = TPS * st, t1 = min(TPS * (st + 1), n_t);
        const uint8_t* kl = lane_k + (st & 1) * C::STAGE;
        const lds_u8* vl = lane_v + (st & 1) * C::STAGE;
        if (t0 < t1) op_s(kl);
        for (int t = t0; t < t1; ++t) {
            // A wave's issue priority falls as it advances through the stage, so the
            // four waves sharing a SIMD keep pace with one another.  Left to age
            // order, the oldest run ahead and the rest finish alone at a fraction of
            // the SIMD's throughput (measured: waves ending 16-28 us into a 31 us
            // launch; with this, 21-26 us into 30 us).
            switch (t - t0) {
                case 0: __builtin_amdgcn_s_setprio(3); break;
                case 1: __builtin_amdgcn_s_setprio(2); break;
                case 2: __builtin_amdgcn_s_setprio(1); break;
                default: __builtin_amdgcn_s_setprio(0); break;
            }
            read_v(vl + (t - t0) * BN * C::VROW);
            op_softmax(t);
            if (t + 1 < t1) op_s(kl + (t + 1 - t0) * BN * C::KROW);
            op_pv();
        }
    }

    // ---- epilogue
    const float l_tot = sum_halves(l_run);
    if (rows && my_q < N) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint8_t* orow = p.o + (slice + static_cast<size_t>(my_q) * D) * 2;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(o[4 * g + e] * inv);
            *reinterpret_cast<bf16x4*>(orow + 2 * (8 * g + 4 * h)) = out;
        }
        if (p.lse != nullptr && h == 0)
            p.lse[static_cast<size_t>(bh) * N + my_q] = (m_run + __log2f(l_tot)) * kLn2;
    }
}

// ===========================================================================
// fp32 kernel: same algorithm on the 32x32x2 fp32 MFMA (no reduced-precision
// products, probabilities kept in fp32 for P*V).
// ===========================================================================
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_f32_kernel(KParams p) {
    constexpr int BM = 128, BN = 32;
    constexpr int KST = D + 1;       // floats per K row in LDS (odd stride: column reads hit distinct banks)
    constexpr int VST = D + 4;       // floats per V row in LDS (16-byte aligned rows)
    constexpr int STAGE = BN * KST + BN * VST;
    constexpr int CHUNKS = BN * D / 4;                 // 16-byte chunks per K (or V) tile
    constexpr int PER_T = (CHUNKS + 255) / 256;
    __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int N = p.N;
    int qt = blockIdx.x / p.BH;
    const int bh = blockIdx.x - qt * p.BH;
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;
    const int q0 = qt * BM, qw0 = q0 + 32 * w, my_q = qw0 + l32;
    const size_t slice = static_cast<size_t>(bh) * N * D;
    const float* qg = reinterpret_cast<const float*>(p.q) + slice;
    const float* kg = reinterpret_cast<const float*>(p.k) + slice;
    const float* vg = reinterpret_cast<const float*>(p.v) + slice;

    float qf[D / 2];                                   // B operand: Q[my_q][2i + h]
#pragma unroll
    for (int i = 0; i < D / 2; ++i) qf[i] = my_q < N ? qg[static_cast<size_t>(my_q) * D + 2 * i + h] : 0.0f;

    const int n_ktiles_all = (N + BN - 1) / BN;
    const int q_end = min(q0 + BM, N);
    const int n_kt = CAUSAL ? min(n_ktiles_all, (q_end + BN - 1) / BN) : n_ktiles_all;

    f32x4 kst[PER_T], vst[PER_T];
    auto load_tile = [&](int j) {
        const int n0 = j * BN;
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int c = i * 256 + tid;
            if (c < CHUNKS) {
                const int row = c / (D / 4), col = c - row * (D / 4);
                const int key = n0 + row;
                const size_t off = static_cast<size_t>(key) * D + 4 * col;
                kst[i] = key < N ? *reinterpret_cast<const f32x4*>(kg + off) : f32x4{0, 0, 0, 0};
                vst[i] = key < N ? *reinterpret_cast<const f32x4*>(vg + off) : f32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&](int buf) {
        float* ks = smem + buf * STAGE;
        float* vs = ks + BN * KST;
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int c = i * 256 + tid;
            if (c < CHUNKS) {
                const int row = c / (D / 4), col = c - row * (D / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) ks[row * KST + 4 * col + e] = kst[i][e];
                *reinterpret_cast<f32x4*>(vs + row * VST + 4 * col) = vst[i];
            }
        }
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] = 0.0f;
    float m_run = kNegInf, l_run = 0.0f;

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int j = 0; j < n_kt; ++j) {
        const int n0 = j * BN;
        const bool more = j + 1 < n_kt;
        if (more) load_tile(j + 1);
        const bool active = !CAUSAL || n0 <= qw0 + 31;
        if (active) {
            const float* ks = smem + (j & 1) * STAGE;
            const float* vs = ks + BN * KST;
            f32x16 acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
            for (int i = 0; i < D / 2; ++i)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[l32 * KST + 2 * i + h], qf[i], acc, 0, 0, 0);
            float s[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] = acc[v];
            if ((CAUSAL && n0 + BN - 1 > qw0) || n0 + BN > N) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = n0 + acc_row(v, h);
                    if (key >= N || (CAUSAL && key > my_q)) s[v] = kNegInf;
                }
            }
            const float alpha = softmax_step(s, p.c_log2, m_run, l_run);
            if (!__all(alpha == 1.0f)) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
            }
            // contraction step v: lane (l32, h) supplies P[my_q][key acc_row(v, h)]
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[acc_row(v, h) * VST + 32 * db + l32], s[v],
                                                                 o[db], 0, 0, 0);
        }
        if (more) store_tile((j + 1) & 1);
        __syncthreads();
    }

    const float l_tot = sum_halves(l_run);
    if (my_q < N) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        float* orow = reinterpret_cast<float*>(p.o) + slice + static_cast<size_t>(my_q) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = o[db][4 * g + e] * inv;
                *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * h) = out;
            }
        if (p.lse != nullptr && h == 0)
            p.lse[static_cast<size_t>(bh) * N + my_q] = (m_run + __log2f(l_tot)) * kLn2;
    }
}

// ===========================================================================
// V -> V^T for the bf16/FP8 kernel (one workgroup per 64-key tile)
//
// P*V needs each lane's eight contracted keys side by side, i.e. V transposed.
// Producing V^T once per call keeps the attention kernel's tile copies plain
// coalesced 16-byte loads and stores.  Within each 64-key tile the keys are
// stored in vt_slot order (the order the P fragments use), and keys >= N are
// zero so padded tiles contribute nothing.
// ===========================================================================
template <int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const uint8_t* __restrict__ v, uint8_t* __restrict__ vt,
                                                          int N, int np, int n_tiles) {
    constexpr int ROW = 2 * D + 16;                // bytes per key row in LDS (padded)
    __shared__ __attribute__((aligned(16))) uint8_t tile[kKeyTile * ROW];
    const int bh = blockIdx.x / n_tiles, t = blockIdx.x - bh * n_tiles;
    const int n0 = kKeyTile * t;
    const uint8_t* src = v + (static_cast<size_t>(bh) * N + n0) * D * 2;
    constexpr int IN_CHUNKS = kKeyTile * D / 8;    // 16-byte chunks of the V tile
    for (int c = threadIdx.x; c < IN_CHUNKS; c += 256) {
        const int key = c / (D / 8), col = c - key * (D / 8);
        const u32x4 x = n0 + key < N ? ld16(src + (key * D + 8 * col) * 2) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(tile + key * ROW + 16 * col) = x;
    }
    __syncthreads();
    uint8_t* dst = vt + (static_cast<size_t>(bh) * D * np + n0) * 2;
    constexpr int OUT_CHUNKS = D * (kKeyTile / 8); // 8 key slots = 16 bytes per chunk
    for (int c = threadIdx.x; c < OUT_CHUNKS; c += 256) {
        const int d = c / (kKeyTile / 8), k8 = c - d * (kKeyTile / 8);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            // vt_slot swaps bits 2 and 3 of the key index, so it is its own inverse
            const int k0 = vt_slot(8 * k8 + e), k1 = vt_slot(8 * k8 + e + 1);
            const uint32_t lo = *reinterpret_cast<const uint16_t*>(tile + k0 * ROW + 2 * d);
            const uint32_t hi = *reinterpret_cast<const uint16_t*>(tile + k1 * ROW + 2 * d);
            w[e >> 1] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(dst + (static_cast<size_t>(d) * np + 8 * k8) * 2) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// ===========================================================================
// Merge of partial results over disjoint key ranges: with M = max_g lse_g,
// lse = M + ln sum_g exp(lse_g - M) and O = sum_g exp(lse_g - lse) O_g (the
// combination step of ring attention, on one device).  D/4 lanes per row,
// four fp32 values of every part per lane.
// ===========================================================================
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_parts, const float* __restrict__ lse_parts,
                                                    int n_parts, uint8_t* __restrict__ o, float* __restrict__ lse,
                                                    long long rows) {
    constexpr int LPR = D / 4;
    const long long row = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) / LPR;
    const int part = threadIdx.x % LPR;
    if (row >= rows) return;
    float m = kNegInf;
    for (int g = 0; g < n_parts; ++g) m = fmaxf(m, lse_parts[g * rows + row]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float lse_out = kNegInf;
    if (m != kNegInf) {
        float wsum = 0.0f;
        for (int g = 0; g < n_parts; ++g) {
            const float wg = expf(lse_parts[g * rows + row] - m);     // 0 for an empty part
            const f32x4 x = *reinterpret_cast<const f32x4*>(o_parts + (g * rows + row) * D + 4 * part);
            wsum += wg;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(wg, x[e], acc[e]);
        }
        const float inv = 1.0f / wsum;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= inv;
        lse_out = m + logf(wsum);
    }
    bf16x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(acc[e]);
    *reinterpret_cast<bf16x4*>(o + (row * D + 4 * part) * 2) = out;
    if (lse != nullptr && part == 0) lse[row] = lse_out;
}

// ===========================================================================
// Per-64-row-tile e4m3fn quantisation (one workgroup per tile)
// ===========================================================================

// e4m3fn code of a finite fp32 value with |y| <= 448, rounded to nearest even.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t bits = __float_as_uint(y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = fabsf(y);
    uint32_t mag;
    if (a < 0.015625f) {
        // below 2^-6 the format is a fixed grid of 2^-9 steps; a count of 8
        // is the smallest normal, whose code is also 8
        mag = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
    } else {
        const uint32_t ab = bits & 0x7FFFFFFFu;
        const uint32_t e = (ab >> 23) - 120u;            // rebias 127 -> 7
        const uint32_t m = ab & 0x7FFFFFu;
        mag = (e << 3) | (m >> 20);
        const uint32_t rem = m & 0xFFFFFu;               // 20 dropped mantissa bits
        mag += (rem > 0x80000u) | ((rem == 0x80000u) & (mag & 1u));
    }
    return sign | mag;
}

__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
                                                        float* __restrict__ scale, int N, int D, int n_tiles) {
    __shared__ float red[4];
    const int tile = blockIdx.x;
    const int bh = tile / n_tiles, t = tile - bh * n_tiles;
    const int r0 = 64 * t;
    const int rows = min(64, N - r0);
    const int n_chunks = rows * D / 8;                   // 8 bf16 per 16-byte chunk
    const size_t base = (static_cast<size_t>(bh) * N + r0) * D;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + base);

    // the whole tile (at most 64 rows x 128 dims: four 16-byte chunks a thread)
    // is loaded at once and kept in registers for the conversion
    constexpr int PER_T = 64 * 128 / 8 / 256;
    u32x4 u[PER_T];
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
        const int c = threadIdx.x + 256 * i;
        u[i] = c < n_chunks ? src[c] : u32x4{0u, 0u, 0u, 0u};
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < PER_T; ++i)
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            amax = fmaxf(amax, fabsf(__uint_as_float(u[i][wd] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(u[i][wd] & 0xFFFF0000u)));
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = 448.0f / fmaxf(amax, 1e-6f);         // IEEE-rounded fp32 division
    if (threadIdx.x == 0) scale[tile] = s;

    u32x2* dst = reinterpret_cast<u32x2*>(x8 + base);
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c >= n_chunks) break;
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t hb = (e & 1) ? (u[i][e >> 1] & 0xFFFF0000u) : (u[i][e >> 1] << 16);
            float y = __uint_as_float(hb) * s;
            y = fminf(fmaxf(y, -448.0f), 448.0f);
            packed[e >> 2] |= e4m3_code(y) << (8 * (e & 3));
        }
        dst[c] = u32x2{packed[0], packed[1]};
    }
}

// ===========================================================================
// e4m3 V^T for the FP8 P*V product: per 64-key tile and column d, the block
// exponent e is the largest integer with amax * 2^e <= 448 (clipped to
// [-127, 127]; 0 for an all-zero column), codes are e4m3(V * 2^e) rounded to
// nearest even, stored transposed with the keys of each tile in f8_slot
// order, and the byte 127 - e (the matrix core's exponent that undoes 2^e)
// goes to vscale [BH, n_tiles, D].
// ===========================================================================
template <int D>
__global__ __launch_bounds__(256) void quant_v_pow2_kernel(const uint8_t* __restrict__ v, uint8_t* __restrict__ v8,
                                                           uint8_t* __restrict__ vscale, int N, int np, int n_tiles) {
    constexpr int ROW = 2 * D + 16;
    constexpr int CPR = D / 8;                     // 16-byte chunks per key row
    constexpr int PER_T = kKeyTile * CPR / 256;    // chunks per thread
    static_assert(PER_T >= 1 && 256 % CPR == 0, "tile split");
    __shared__ __attribute__((aligned(16))) uint8_t tile[kKeyTile * ROW];
    __shared__ float wmax[4][D];                   // per-wave column maxima
    __shared__ int sexp[D];
    const int bh = blockIdx.x / n_tiles, t = blockIdx.x - bh * n_tiles;
    const int n0 = kKeyTile * t;
    const uint8_t* src = v + (static_cast<size_t>(bh) * N + n0) * D * 2;
    // every chunk of the tile is loaded at once; a thread's chunks share one
    // column group (dims 8 col ..), whose magnitudes it folds into pm as they go
    // to LDS
    const int col = static_cast<int>(threadIdx.x) % CPR;
    u32x4 x[PER_T];
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
        const int key = (static_cast<int>(threadIdx.x) + 256 * i) / CPR;
        x[i] = n0 + key < N ? ld16(src + (key * D + 8 * col) * 2) : u32x4{0, 0, 0, 0};
    }
    float pm[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
        const int key = (static_cast<int>(threadIdx.x) + 256 * i) / CPR;
        *reinterpret_cast<u32x4*>(tile + key * ROW + 16 * col) = x[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t hb = (e & 1) ? (x[i][e >> 1] & 0xFFFF0000u) : (x[i][e >> 1] << 16);
            pm[e] = fmaxf(pm[e], fabsf(__uint_as_float(hb)));
        }
    }
    // lanes of a wave with the same column group, then the four waves
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) pm[e] = fmaxf(pm[e], __shfl_xor(pm[e], off));
    if ((threadIdx.x & 63) < CPR) {
#pragma unroll
        for (int e = 0; e < 8; ++e) wmax[threadIdx.x >> 6][8 * col + e] = pm[e];
    }
    __syncthreads();
    auto val = [&](int key, int d) -> float {
        return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(tile + key * ROW + 2 * d)) << 16);
    };
    for (int d = threadIdx.x; d < D; d += 256) {
        const float amax = fmaxf(fmaxf(wmax[0][d], wmax[1][d]), fmaxf(wmax[2][d], wmax[3][d]));
        int e = 0;
        if (amax > 0.0f) {
            int x;
            const float m = frexpf(amax, &x);              // amax = m * 2^x, m in [0.5, 1); 448 = 0.875 * 2^9
            e = m <= 0.875f ? 9 - x : 8 - x;
            e = e > 127 ? 127 : (e < -127 ? -127 : e);
        }
        sexp[d] = e;
        vscale[(static_cast<size_t>(bh) * n_tiles + t) * D + d] = static_cast<uint8_t>(127 - e);
    }
    __syncthreads();
    uint8_t* dst = v8 + static_cast<size_t>(bh) * D * np + n0;
    for (int c = threadIdx.x; c < D * (kKeyTile / 16); c += 256) {
        const int d = c / (kKeyTile / 16), part = c - d * (kKeyTile / 16);
        const int e = sexp[d];
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int pos = 16 * part + i;
            // inverse of f8_slot
            const int key = (((pos >> 4) & 1) << 5) | (((pos >> 2) & 3) << 3) | (((pos >> 5) & 1) << 2) | (pos & 3);
            const uint32_t code = e4m3_code(ldexpf(val(key, d), e));
            w[i >> 2] |= code << (8 * (i & 3));
        }
        *reinterpret_cast<u32x4*>(dst + static_cast<size_t>(d) * np + 16 * part) = u32x4{w[0], w[1], w[2], w[3]};
    }
}


template <bool CAUSAL, bool FP8, bool PV8 = false>
hipError_t launch_b128(KParams kp, int BH, hipStream_t st) {
    using C = B128Cfg<FP8, PV8>;
    kp.n_qtiles = (kp.N + C::BM - 1) / C::BM;
    // XCD-banded order where every XCD gets the same heads: bands of as many of
    // an XCD's heads as keep their K and V within 8 MiB (twice one XCD's L2:
    // the band's query tiles stream them roughly in step), if that is at least
    // two.  (Measured at 4x32x4096x128 causal, 2 MiB of K and V per head: bands
    // of 1 / 2 / 4 / 8 heads +2.5 / -1.9 / -3.0 / -2.5 % against query-tile
    // major; at 1x32x16384x128, 8 MiB per head: bands of 1 +0.9 %.)
    kp.band = 0;
    if (BH % kXcds == 0) {
        const int per_xcd = BH / kXcds;
        const long long kv = static_cast<long long>(kp.N) * C::D * (C::ES + (PV8 ? 1 : 2));
        int band = static_cast<int>(std::min<long long>(per_xcd, (8LL << 20) / kv));
        while (band > 1 && per_xcd % band != 0) --band;
        kp.band = band >= 2 ? band : 0;
    }
    const long long grid = static_cast<long long>(kp.n_qtiles) * BH;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_b128_kernel<CAUSAL, FP8, PV8>), dim3(static_cast<int>(grid)), dim3(C::NT), 0, st, kp);
    return hipGetLastError();
}

template <bool CAUSAL>
hipError_t launch_d32(KParams kp, int BH, hipStream_t st) {
    using C = D32Cfg<256>;
    // workgroups per head: 256-query tiles, or (causal) pairs of 128-query chunks
    kp.n_qtiles = CAUSAL ? ((kp.N + 127) / 128 + 1) / 2 : (kp.N + C::BM - 1) / C::BM;
    const long long grid = static_cast<long long>(kp.n_qtiles) * BH;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_d32_kernel<CAUSAL, 256>), dim3(static_cast<int>(grid)), dim3(C::NT), 0, st, kp);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool FP8>
hipError_t launch_bf(KParams kp, int BH, hipStream_t st) {
    if constexpr (D == 128) {
        return launch_b128<CAUSAL, FP8>(kp, BH, st);
    } else if constexpr (D == 32 && !FP8) {
        return launch_d32<CAUSAL>(kp, BH, st);
    } else {
        kp.n_qtiles = (kp.N + PPCfg<D, CAUSAL, FP8>::BM - 1) / PPCfg<D, CAUSAL, FP8>::BM;
        const long long grid = static_cast<long long>(kp.n_qtiles) * BH;
        if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((fwd_pp_kernel<D, CAUSAL, FP8, kModeDense>), dim3(static_cast<int>(grid)),
                           dim3(PPCfg<D, CAUSAL, FP8>::NT), 0, st, kp);
        return hipGetLastError();
    }
}
template <int D, bool CAUSAL>
hipError_t launch_fp8pv(KParams kp, int BH, hipStream_t st) {
    if constexpr (D == 128) return launch_b128<CAUSAL, true, true>(kp, BH, st);
    using C = PPCfg<D, CAUSAL, true, true>;
    kp.n_qtiles = (kp.N + C::BM - 1) / C::BM;
    const long long grid = static_cast<long long>(kp.n_qtiles) * BH;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_pp_kernel<D, CAUSAL, true, kModeDense, true>), dim3(static_cast<int>(grid)), dim3(C::NT),
                       0, st, kp);
    return hipGetLastError();
}
template <int D, bool CAUSAL>
hipError_t launch_partial(KParams kp, int BH, hipStream_t st) {
    kp.n_qtiles = (kp.N + PPCfg<D, CAUSAL, false>::BM - 1) / PPCfg<D, CAUSAL, false>::BM;
    const long long grid = static_cast<long long>(kp.n_qtiles) * BH * kp.n_splits;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_pp_kernel<D, CAUSAL, false, kModePartial>), dim3(static_cast<int>(grid)),
                       dim3(PPCfg<D, CAUSAL, false>::NT), 0, st, kp);
    return hipGetLastError();
}
template <int D, bool CAUSAL>
hipError_t launch_sparse(KParams kp, int BH, hipStream_t st) {
    static_assert(PPCfg<D, CAUSAL, false>::BM == kQueryTile, "visit lists are planned per 256-query tile");
    kp.n_qtiles = (kp.N + PPCfg<D, CAUSAL, false>::BM - 1) / PPCfg<D, CAUSAL, false>::BM;
    const long long grid = static_cast<long long>(kp.n_qtiles) * BH;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_pp_kernel<D, CAUSAL, false, kModeSparse>), dim3(static_cast<int>(grid)),
                       dim3(PPCfg<D, CAUSAL, false>::NT), 0, st, kp);
    return hipGetLastError();
}

// Visit lists of the block-sparse kernel: one thread per (bh, 256-query tile)
// walks the key tiles and keeps those that one of its four 64-query blocks
// may see (table entry set, and at or below the diagonal when causal).
__global__ __launch_bounds__(256) void bs_plan_kernel(const uint8_t* __restrict__ mask, long long mask_bh_stride,
                                                      int BH, int n_qtiles, int nb, bool causal,
                                                      uint32_t* __restrict__ list, int* __restrict__ count) {
    const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<long long>(BH) * n_qtiles) return;
    const int bh = static_cast<int>(idx / n_qtiles), qt = static_cast<int>(idx - static_cast<long long>(bh) * n_qtiles);
    const uint8_t* mb = mask + static_cast<size_t>(bh) * mask_bh_stride;
    uint32_t* out = list + static_cast<size_t>(idx) * nb;
    int cnt = 0;
    for (int kb = 0; kb < nb; ++kb) {
        uint32_t flags = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int qb = 4 * qt + b;
            if (qb < nb && mb[static_cast<size_t>(qb) * nb + kb] != 0 && (!causal || kb <= qb)) flags |= 1u << b;
        }
        if (flags != 0) out[cnt++] = static_cast<uint32_t>(kb) | (flags << 24);
    }
    count[idx] = cnt;
}
template <int D, bool CAUSAL>
hipError_t launch_f32(KParams kp, int BH, hipStream_t st) {
    kp.n_qtiles = (kp.N + 127) / 128;
    const long long grid = static_cast<long long>(kp.n_qtiles) * BH;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(static_cast<int>(grid)), dim3(256), 0, st, kp);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_d(const FwdArgs& a, const KParams& kp, hipStream_t st) {
    const int BH = a.BH;
    if (a.o32 != nullptr)
        return a.causal ? launch_partial<D, true>(kp, BH, st) : launch_partial<D, false>(kp, BH, st);
    if (a.bs_list != nullptr)
        return a.causal ? launch_sparse<D, true>(kp, BH, st) : launch_sparse<D, false>(kp, BH, st);
    switch (a.kind) {
        case Kind::F32:
            return a.causal ? launch_f32<D, true>(kp, BH, st) : launch_f32<D, false>(kp, BH, st);
        case Kind::BF16:
            return a.causal ? launch_bf<D, true, false>(kp, BH, st) : launch_bf<D, false, false>(kp, BH, st);
        case Kind::FP8:
            return a.causal ? launch_bf<D, true, true>(kp, BH, st) : launch_bf<D, false, true>(kp, BH, st);
        case Kind::FP8PV:
            return a.causal ? launch_fp8pv<D, true>(kp, BH, st) : launch_fp8pv<D, false>(kp, BH, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    KParams kp;
    kp.q = static_cast<const uint8_t*>(a.q);
    kp.k = static_cast<const uint8_t*>(a.k);
    kp.v = static_cast<const uint8_t*>(a.v);
    kp.vt = static_cast<const uint8_t*>(a.vt);
    kp.np = a.np;
    kp.o = static_cast<uint8_t*>(a.o);
    kp.lse = a.lse;
    kp.q_scale = a.q_scale;
    kp.k_scale = a.k_scale;
    kp.BH = a.BH;
    kp.N = a.N;
    kp.n_qtiles = 0;                       // set per kernel from its query-tile height
    kp.c_log2 = a.softmax_scale * kLog2e;
    kp.o32 = a.o32;
    kp.lse_part = a.lse_part;
    kp.kt_lo = a.kt_lo;
    kp.kt_hi = a.kt_hi;
    kp.tps = a.tps;
    kp.n_splits = a.n_splits;
    kp.bs_list = a.bs_list;
    kp.bs_count = a.bs_count;
    kp.bs_stride = a.bs_stride;
    kp.vscale = a.v_scale;
    kp.band = 0;
    if (a.kind == Kind::FP8PV && (a.v_scale == nullptr || a.o32 != nullptr || a.bs_list != nullptr))
        return hipErrorInvalidValue;
    if (a.o32 != nullptr && (a.kind != Kind::BF16 || a.n_splits < 1 || a.tps < 1)) return hipErrorInvalidValue;
    if (a.bs_list != nullptr && (a.kind != Kind::BF16 || a.o32 != nullptr)) return hipErrorInvalidValue;
    switch (a.d) {
        case 32: return dispatch_d<32>(a, kp, stream);
        case 64: return dispatch_d<64>(a, kp, stream);
        case 128: return dispatch_d<128>(a, kp, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_transpose_v(const void* v, void* vt, int BH, int N, int d, hipStream_t stream) {
    const int n_tiles = (N + kKeyTile - 1) / kKeyTile;
    const int np = n_tiles * kKeyTile;
    const long long grid = static_cast<long long>(BH) * n_tiles;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    const uint8_t* src = static_cast<const uint8_t*>(v);
    uint8_t* dst = static_cast<uint8_t*>(vt);
    switch (d) {
        case 32: hipLaunchKernelGGL(transpose_v_kernel<32>, dim3(static_cast<int>(grid)), dim3(256), 0, stream, src, dst, N, np, n_tiles); break;
        case 64: hipLaunchKernelGGL(transpose_v_kernel<64>, dim3(static_cast<int>(grid)), dim3(256), 0, stream, src, dst, N, np, n_tiles); break;
        case 128: hipLaunchKernelGGL(transpose_v_kernel<128>, dim3(static_cast<int>(grid)), dim3(256), 0, stream, src, dst, N, np, n_tiles); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bs_plan(const uint8_t* mask, long long mask_bh_stride, int BH, int N, bool causal,
                          uint32_t* list, int* count, hipStream_t stream) {
    const int nb = (N + kKeyTile - 1) / kKeyTile;
    const int n_qtiles = (N + 255) / 256;
    const long long threads = static_cast<long long>(BH) * n_qtiles;
    const long long grid = (threads + 255) / 256;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bs_plan_kernel, dim3(static_cast<int>(grid)), dim3(256), 0, stream, mask, mask_bh_stride, BH,
                       n_qtiles, nb, causal, list, count);
    return hipGetLastError();
}

hipError_t launch_quant_v_pow2(const void* v, uint8_t* v8, uint8_t* vscale, int BH, int N, int d,
                              hipStream_t stream) {
    const int n_tiles = (N + kKeyTile - 1) / kKeyTile;
    const int np = n_tiles * kKeyTile;
    const long long grid = static_cast<long long>(BH) * n_tiles;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    const uint8_t* src = static_cast<const uint8_t*>(v);
    switch (d) {
        case 32: hipLaunchKernelGGL(quant_v_pow2_kernel<32>, dim3(static_cast<int>(grid)), dim3(256), 0, stream, src, v8, vscale, N, np, n_tiles); break;
        case 64: hipLaunchKernelGGL(quant_v_pow2_kernel<64>, dim3(static_cast<int>(grid)), dim3(256), 0, stream, src, v8, vscale, N, np, n_tiles); break;
        case 128: hipLaunchKernelGGL(quant_v_pow2_kernel<128>, dim3(static_cast<int>(grid)), dim3(256), 0, stream, src, v8, vscale, N, np, n_tiles); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse,
                        int BH, int N, int d, hipStream_t stream) {
    const long long rows = static_cast<long long>(BH) * N;
    const long long grid = (rows * (d / 4) + 255) / 256;
    if (grid > 0x7FFFFFFFLL || n_parts < 1) return hipErrorInvalidConfiguration;
    uint8_t* out = static_cast<uint8_t*>(o);
    switch (d) {
        case 32: hipLaunchKernelGGL(merge_kernel<32>, dim3(static_cast<int>(grid)), dim3(256), 0, stream, o_parts, lse_parts, n_parts, out, lse, rows); break;
        case 64: hipLaunchKernelGGL(merge_kernel<64>, dim3(static_cast<int>(grid)), dim3(256), 0, stream, o_parts, lse_parts, n_parts, out, lse, rows); break;
        case 128: hipLaunchKernelGGL(merge_kernel<128>, dim3(static_cast<int>(grid)), dim3(256), 0, stream, o_parts, lse_parts, n_parts, out, lse, rows); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quant_fp8(const void* x_bf16, uint8_t* x8, float* scale, int BH, int N, int d,
                            hipStream_t stream) {
    const int n_tiles = (N + 63) / 64;
    const long long grid = static_cast<long long>(BH) * n_tiles;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    if (d > 128 || d % 8 != 0) return hipErrorInvalidValue;    // a tile is at most four chunks a thread
    hipLaunchKernelGGL(quant_fp8_kernel, dim3(static_cast<int>(grid)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x_bf16), x8, scale, N, d, n_tiles);
    return hipGetLastError();
}

}  // namespace fa
