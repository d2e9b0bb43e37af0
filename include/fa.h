/*
 * fa.h -- C ABI of fused attention (forward and backward) for MI355X (gfx950).
 *
 * The main operation is FlashAttention's forward pass:
 *
 *     O   = softmax(softmax_scale * Q K^T  [causally masked]) V
 *     lse = per-row natural log of the softmax denominator, i.e.
 *           lse_i = ln sum_j exp(softmax_scale * q_i . k_j) over unmasked j
 *
 * computed tile by tile with an online softmax (running max m and running
 * sum l, partial O rescaled as the max grows), so the N x N score matrix
 * never reaches device memory.  Pages defining it:
 *   - "Flash Attention" tag page (guijiagi.com): excerpt on what
 *     FlashAttention solves (S = QK^T/sqrt(d), P = softmax(S), O = PV), the
 *     excerpt on the performance bottleneck (online softmax over blocks,
 *     deferred rescale, parallelism over batch and heads) and the standard
 *     attention listing ((batch, heads, seq, dim) layout);
 *   - "From theory to implementation: the three FlashAttention generations
 *     dissected with Triton": section 2.1 (running max / sum update),
 *     3.1 (per-block causal mask), 4.1 (FP8 with dynamic per-block scales);
 *   - "Core principles behind FlashAttention's speed-up": section 1.2
 *     (one fused kernel), 1.3 (online renormalisation), 4.2
 *     (softmax_scale, conventionally 1/sqrt(dim)).
 *
 * fa_bwd is its gradient: dQ, dK, dV for an upstream gradient dO, with the
 * probabilities recomputed from Q, K and the forward's lse instead of stored
 * (Triton walkthrough page, section 2.2).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, contiguous, row-major [B, H, N, d] (batch, heads,
 *     sequence, head dim) in device memory.  Base pointers of q, k, v, o,
 *     q8, k8 must be 16-byte aligned; lse and scale pointers 4-byte aligned.
 *   - Supported head dims: d in {32, 64, 128}.  Any N >= 1 (tails are
 *     masked); B, H >= 1; B*H*ceil(N/64)*64*d < 2^31.
 *   - Causal masking keeps key j for query i iff j <= i (square attention,
 *     Nq = Nk = N).
 *   - lse is float32 [B, H, N] and may be NULL (then it is not written).
 *   - The caller owns every buffer; the library never frees or keeps them.
 *     o must not alias q, k or v.  No state is kept between calls; calls on
 *     different streams may run concurrently.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     on it and the call returns without synchronising; faults during
 *     execution surface at the caller's next synchronisation on it.
 *     A call makes no memset, host read-back or synchronising HIP call, so
 *     it may be captured into a HIP graph (the workspaces become the
 *     graph's allocation nodes).
 *   - Arguments are validated before any HIP call, so argument errors are
 *     reported synchronously (also on a machine with no GPU).  No
 *     exceptions, aborts or prints cross this ABI.
 *   - A call whose stream-ordered workspace cannot be allocated returns
 *     FA_ERR_OUT_OF_MEMORY having enqueued nothing.  Setting the environment
 *     variable FA_TEST_FAIL_ALLOC=1 makes every workspace request fail this
 *     way (read at each call; for tests of that path).
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 6

/* Size of the static device buffer behind fa_fwd_splitkv_noalloc (per GPU). */
#define FA_NOALLOC_SCRATCH_BYTES (128u << 20)

typedef enum {
    FA_F32 = 0,       /* q, k, v, o float32; products and softmax in fp32 */
    FA_BF16 = 1,      /* q, k, v, o bfloat16; fp32 accumulation */
    FA_FP8_E4M3 = 2,  /* q, k, v, o bfloat16 on input; Q and K quantised to
                         e4m3fn per 64-row tile inside the call (see
                         fa_quant_fp8_e4m3), V and P*V stay bf16 */
    FA_FP8_E4M3_PV = 3, /* as FA_FP8_E4M3, and P*V also on e4m3 matrix cores:
                         V quantised per (64-key tile, column) with a
                         power-of-two scale (see fa_quant_v_pow2), P per
                         (query, 64-key tile) with a power-of-two scale
                         inside the kernel; both scales are the MFMA's own
                         block exponents, so dequantisation is exact.  V
                         must be finite: at d = 128, when N mod 128 lies in
                         1..64, the missing half of the last 128-key tile
                         meets the next V^T row's codes with P = 0, and a
                         NaN there would reach another column of O */
    /* not dtypes: they widen the enumeration so that any int a caller
       passes is a valid value of it (reported as FA_ERR_INVALID_DTYPE) */
    FA_DTYPE_MIN_ENUM = -0x7FFFFFFF - 1,
    FA_DTYPE_MAX_ENUM = 0x7FFFFFFF
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL_POINTER = 1,
    FA_ERR_INVALID_SHAPE = 2,
    FA_ERR_UNSUPPORTED_HEAD_DIM = 3,
    FA_ERR_INVALID_SCALE = 4,
    FA_ERR_INVALID_DTYPE = 5,
    FA_ERR_MISALIGNED = 6,
    FA_ERR_INVALID_ARGUMENT = 7,
    FA_ERR_UNSUPPORTED_ARCH = 8,
    FA_ERR_OUT_OF_MEMORY = 9,
    FA_ERR_LAUNCH = 10,
    FA_ERR_HIP = 11,
    FA_ERR_SCRATCH_LIMIT = 12,    /* problem too large for fa_fwd_splitkv_noalloc */
    /* not statuses: any int is a valid value of the enumeration */
    FA_STATUS_MIN_ENUM = -0x7FFFFFFF - 1,
    FA_STATUS_MAX_ENUM = 0x7FFFFFFF
} fa_status;

/*
 * fa_fwd -- fused attention forward.
 *   q, k, v : inputs [B,H,N,d] of the element type named by `dtype`.
 *   o       : output [B,H,N,d], same element type as q (bf16 for FP8).
 *   lse     : output float32 [B,H,N] or NULL.
 *   causal  : 0 or 1.
 *   softmax_scale : finite and > 0; multiplies the fp32 scores (it is not
 *             folded into the stored Q).
 *   dtype   : FA_F32, FA_BF16, FA_FP8_E4M3 or FA_FP8_E4M3_PV.  FA_F32 and
 *             FA_BF16 run one kernel and allocate nothing.  FA_FP8_E4M3
 *             allocates one stream-ordered workspace (hipMallocAsync /
 *             hipFreeAsync on `stream`) for the quantised Q, K and their
 *             scales (it runs fa_quant_fp8_e4m3 on q and k before the FP8
 *             kernel); FA_FP8_E4M3_PV also for the e4m3 V^T and its
 *             exponents (fa_quant_v_pow2).
 * Returns FA_OK or the first error found.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t N, int64_t d,
                 int causal, float softmax_scale, fa_dtype dtype, void* stream);

/*
 * fa_quant_fp8_e4m3 -- per-tile dynamic FP8 quantisation (Triton walkthrough
 * page, section 4.1: a scale from the block's largest magnitude; here with
 * the e4m3fn range 448 and 64-row tiles).
 *   x_bf16 : input bf16 [BH, N, d] (BH = B*H independent slices).
 *   x8     : output e4m3fn codes, bytes [BH, N, d].
 *   scale  : output float32 [BH, ceil(N/64)].
 * For every slice and tile t of rows [64t, min(64t+64, N)):
 *   amax = max |x| over the tile;  scale_t = 448.0f / max(amax, 1e-6f)
 *   (IEEE fp32 division);  code = e4m3fn_RNE(clamp(fp32(x * scale_t), +-448)).
 * Dequantisation is x ~= decode(code) / scale_t.
 */
fa_status fa_quant_fp8_e4m3(const void* x_bf16, uint8_t* x8, float* scale,
                            int64_t BH, int64_t N, int64_t d, void* stream);

/*
 * fa_quant_v_pow2 -- the V pre-pass of FA_FP8_E4M3_PV (tag page, excerpt on
 * V3: FP8 for the products; the power-of-two scale is this library's reading).
 *   v_bf16  : input bf16 [BH, N, d].
 *   v8      : output e4m3fn codes [BH, d, np] with np = ceil(N/64)*64: V
 *             transposed, the 64 keys of each tile stored in the order the
 *             attention kernel's P operand meets them, padding codes 0.
 *   v_scale : output bytes [BH, ceil(N/64), d]: 127 - e, where e is the
 *             largest integer (clipped to [-127, 127]; 0 for an all-zero
 *             column) with max|V| over the tile's keys in that column * 2^e
 *             <= 448.  code = e4m3fn_RNE(V * 2^e); V ~= decode(code) * 2^-e.
 */
fa_status fa_quant_v_pow2(const void* v_bf16, uint8_t* v8, uint8_t* v_scale, int64_t BH, int64_t N, int64_t d,
                          void* stream);

/*
 * fa_fwd_fp8 -- attention forward on already-quantised Q and K.
 *   q8, k8   : e4m3fn codes [B,H,N,d];  q_scale, k_scale : float32
 *              [B,H,ceil(N/64)] as written by fa_quant_fp8_e4m3.
 *   v_bf16   : bf16 [B,H,N,d];  o_bf16 : bf16 output [B,H,N,d];  lse as above.
 * Scores are softmax_scale * (q8 . k8) / (q_scale[i/64] * k_scale[j/64])
 * (Triton walkthrough page, section 4.1: the dequantisation multiplies the
 * scores by 1/(q_scale * k_scale)), the products taken on e4m3 matrix cores,
 * which add each run of 8 products aligned to the largest with about 14
 * significant bits and accumulate those sums in fp32.  Allocates nothing.
 */
fa_status fa_fwd_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                     const void* v_bf16, void* o_bf16, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d,
                     int causal, float softmax_scale, void* stream);

/*
 * fa_fwd_partial -- attention of every query over one key range only (bf16),
 * the per-shard step of ring attention ("Flash Attention" tag page,
 * excerpts on attention variants and on ring attention: the sequence is
 * split over devices, each computes local attention and partial results are
 * passed on and combined).
 *   q, k, v : bf16 [B,H,N,d].  Keys [kv_begin, kv_end) are used, at their
 *             positions in the sequence (the causal mask compares them with
 *             the query positions 0..N-1 as they are).
 *   kv_begin: multiple of 64;  kv_end: multiple of 64 or N;
 *             0 <= kv_begin <= kv_end <= N (else FA_ERR_INVALID_ARGUMENT).
 *   o_part  : float32 [B,H,N,d] output: O normalised over the visible keys of
 *             the range (0 for a row that sees none of them).
 *   lse_part: float32 [B,H,N] output: ln of the range's softmax denominator
 *             (-inf for a row that sees none of its keys).
 * Allocates nothing.
 */
fa_status fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                         int64_t B, int64_t H, int64_t N, int64_t d, int64_t kv_begin, int64_t kv_end,
                         int causal, float softmax_scale, void* stream);

/*
 * fa_merge -- combine n_parts partial results over disjoint key ranges.
 *   o_parts : float32 [n_parts, B,H,N,d];  lse_parts : float32 [n_parts, B,H,N]
 *             (as written by fa_fwd_partial; 1 <= n_parts <= 1024).
 *   o       : bf16 output [B,H,N,d];  lse : float32 [B,H,N] output or NULL.
 * With M = max_g lse_g:  lse = M + ln sum_g exp(lse_g - M),
 *                        O   = sum_g exp(lse_g - lse) O_g
 * (a row whose parts are all -inf gets O = 0 and lse = -inf).  Allocates
 * nothing.
 */
fa_status fa_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, void* o, float* lse,
                   int64_t B, int64_t H, int64_t N, int64_t d, void* stream);

/*
 * fa_fwd_splitkv -- fa_fwd for bf16 with the keys of every (b, h) split into
 * n_splits ranges of whole 64-key tiles that run as separate workgroups,
 * then merged as by fa_merge (1 <= n_splits <= 1024).  Same result as
 * fa_fwd up to rounding; it fills the device when B*H*ceil(N/256) is small.
 * Allocates one stream-ordered workspace: n_splits float32 partial O and
 * lse (n_splits*B*H*N*(d+1)*4 bytes).
 */
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t N, int64_t d, int causal, float softmax_scale,
                         int64_t n_splits, void* stream);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, kernels and results (bit for bit)
 * as fa_fwd_splitkv, but the partial O and lse live in a static device buffer
 * of the library, FA_NOALLOC_SCRATCH_BYTES (128 MiB) on each GPU it runs on,
 * held until the process ends.  The call makes no hipMalloc, hipFree or
 * memset; the caller still passes the inputs and o / lse.
 *   Limit: n_splits*B*H*N*d*4 + n_splits*B*H*N*4 bytes, each part rounded up
 *   to 256, must not exceed FA_NOALLOC_SCRATCH_BYTES, else
 *   FA_ERR_SCRATCH_LIMIT (checked before any HIP call).
 *   Every call on one GPU uses that GPU's single buffer, which keeps the last
 *   call's contents (nothing in it needs clearing: a call writes every entry
 *   it reads).  Calls that overlap on one GPU -- on several streams, or from
 *   several host threads -- race on it and give wrong results: serialise them.
 */
fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int64_t B, int64_t H, int64_t N, int64_t d, int causal, float softmax_scale,
                                 int64_t n_splits, void* stream);

/*
 * fa_fwd_blocksparse -- bf16 attention where only the blocks a 0/1 table
 * allows are computed ("Flash Attention" tag page, excerpt on attention
 * variants: block sparse attention cuts the attention matrix into blocks
 * and computes only some of them).
 *   q, k, v, o, lse : as fa_fwd with FA_BF16 (lse may be NULL).
 *   block_mask : device bytes; with nb = ceil(N/64), key j is visible to
 *             query i iff block_mask[(b*H + h)*mask_bh_stride + (i/64)*nb + j/64]
 *             != 0 (and j <= i when causal = 1).
 *   mask_bh_stride : 0 (one nb x nb table for every (b, h)) or nb*nb (one
 *             table per (b, h)); anything else is FA_ERR_INVALID_ARGUMENT.
 * A row that sees no key gets O = 0 and lse = -inf.  Key tiles that no
 * query of a 256-row tile may see are never loaded.  Allocates one
 * stream-ordered workspace for the per-tile visit lists
 * (B*H*ceil(N/256)*(nb+1)*4 bytes).
 */
fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t N, int64_t d, const uint8_t* block_mask,
                             int64_t mask_bh_stride, int causal, float softmax_scale, void* stream);

/*
 * fa_bwd -- gradient of fa_fwd (FA_BF16 only).
 *   q, k, v : the forward's bf16 inputs [B,H,N,d].
 *   o       : the forward's bf16 output [B,H,N,d].
 *   dout    : bf16 upstream gradient dL/dO [B,H,N,d].
 *   lse     : float32 [B,H,N] as written by fa_fwd for the same inputs
 *             (required, not NULL).
 *   dq, dk, dv : bf16 outputs [B,H,N,d]; must not alias any input.
 *   causal, softmax_scale : as given to fa_fwd.
 *   dtype   : FA_BF16 (anything else returns FA_ERR_INVALID_DTYPE).
 * With P = exp(softmax_scale * Q K^T [masked] - lse):
 *   dV = P^T dO;  dP = dO V^T;  D_i = sum_k dO_ik O_ik;  dS = P * (dP - D);
 *   dQ = softmax_scale * dS K;  dK = softmax_scale * dS^T Q.
 * P and dS are rounded to bf16 for the matrix cores; accumulation is fp32.
 * The call allocates one stream-ordered workspace (hipMallocAsync /
 * hipFreeAsync on `stream`): two float32 [B,H,N] row statistics and, for
 * d = 32 and 64 only, Q, dO and K transposed (3*B*H*d*ceil(N/64)*64 bf16;
 * at d = 128 the kernels read those operands out of the natural rows).
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv,
                 int64_t B, int64_t H, int64_t N, int64_t d,
                 int causal, float softmax_scale, fa_dtype dtype, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_string(fa_status s);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
