/*
 * qlin.h -- C ABI of the MI355X (gfx950) weight-quantized decode linear layer
 *
 *     y[M,N] = dequant(W[N,K]) . x[M,K],   M = 1..16 tokens
 *
 * in four variants: W8A8 INT8, FP8-E4M3 weight-only (and FP8 W8A8 with
 * E4M3 / E5M2 codes), 128x128 block-scaled FP8 with UE8M0 scales, and the
 * MXFP4 expert GEMV behind top-k routing (also as a routed expert FFN).
 *
 * Sources (web pages, by title and section):
 *   [Z100] "Hygon Z100 (gfx906) vLLM adaptation: optimisation and operator
 *          development record (condensed)", chapter 2 (hand-written HIP
 *          operators): operator-family table; 2.1 INT8 W8A8 sdot4; 2.2 FP8
 *          emulation; 2.4 block-scaled (128x128) FP8 extension; pitfall 6 of
 *          section 3 (padded weight row stride).
 *   [DSV4] "vLLM 0.27.x port: DeepSeek V4 Flash FP4 on Hygon DCU gfx936,
 *          full report": 3.3 quantisation config; 7.4 UE8M0 decode;
 *          9.3 MXFP4 MoE emulation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *   never allocates, frees or synchronises: each call only enqueues kernels
 *   on `stream` (a hipStream_t passed as void*; NULL = the null stream) and
 *   returns.  Calls are stateless and thread-safe; two calls that write the
 *   same output buffer race like any two kernels would.
 * - Matrices are row-major.  A row pitch `ld*` is counted in ELEMENTS of the
 *   stored type (bytes for int8 / E4M3 / UE8M0 codes, 2-byte units for bf16).
 *   Weights are [N, K] with K contiguous, used exactly as stored; a padded
 *   row pitch ldw > K is accepted (the padded view reads the same values as
 *   the contiguous one), an unsupported stride is an error, never a copy.
 * - bf16 values are IEEE binary32 with the low 16 bits dropped; outputs are
 *   rounded to nearest, ties to even.
 * - Return value: QLIN_OK (0) or a negative QLIN_ERR_* code.  Every argument
 *   error is detected on the host BEFORE anything is enqueued, and then no
 *   output is touched.  QLIN_ERR_LAUNCH reports a HIP launch failure.
 * - Device-resident data is not validated (that would need a host sync):
 *   NaN/Inf inputs give unspecified outputs; see each call for the rest.
 * - M (tokens): the dense entry points (INT8, FP8, FP8 W8A8, block FP8 and
 *   their quantisers) and qlin_moe_mxfp4 accept 1 <= M <= QLIN_MAX_M_PREFILL;
 *   up to 16 they run the decode kernels, above 16 a tiled (grouped, for
 *   the MoE) matrix-core GEMM with the same arithmetic contract.  The routed
 *   expert FFN and the per-tensor FP8 quantiser take 1 <= M <= QLIN_MAX_M.
 * - Base pointers and row pitches of weights, codes and bf16 activations must
 *   be 16-byte aligned (128-bit loads); scale arrays must be naturally
 *   aligned.
 */
#ifndef QLIN_H
#define QLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    QLIN_OK = 0,
    QLIN_ERR_NULL = -1,      /* a required pointer is NULL */
    QLIN_ERR_SHAPE = -2,     /* M, N, K or topk outside the supported range / multiple */
    QLIN_ERR_STRIDE = -3,    /* a row pitch is smaller than the row it must hold */
    QLIN_ERR_ALIGN = -4,     /* a base pointer or row pitch breaks the alignment rule */
    QLIN_ERR_WORKSPACE = -5, /* workspace missing or smaller than required */
    QLIN_ERR_ARG = -6,       /* an enum/flag argument has an unknown value */
    QLIN_ERR_LAUNCH = -7     /* HIP reported an error when enqueuing a kernel */
};

#define QLIN_MAX_M 16
#define QLIN_MAX_M_PREFILL 16384

/* FP8 code formats (OCP 8-bit floating point) of the W8A8 FP8 entry points. */
enum {
    QLIN_FMT_E4M3 = 0, /* e4m3fn: bias 7, no infinities, largest finite 448 */
    QLIN_FMT_E5M2 = 1  /* e5m2: bias 15, +-inf and NaN, largest finite 57344 */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* qlin_status_str(int status);

/* Library version as an integer (major*10000 + minor*100 + patch). */
int qlin_version(void);

/* ------------------------------------------------------------------------
 * (a) W8A8 INT8 -- [Z100] operator-family table (INT8 row) and section 2.1
 * ------------------------------------------------------------------------ */

/* Dynamic per-token symmetric INT8 activation quantisation.
 *   x   bf16 [M, ldx]   input activations (row pitch ldx >= K)
 *   xq  int8 [M, ldxq]  output codes:  q = clamp(rne(x / s), -127, 127)
 *   xs  fp32 [M]        output scales: s = max_k |x[m,k]| / 127
 * Both divisions are IEEE fp32 with round-to-nearest-even; rne rounds half
 * to even.  A token whose row is all zero gets s = 0 and codes 0.
 * Requires K % 16 == 0, 16 <= K <= 131072, ldx % 8 == 0, ldxq % 16 == 0. */
int qlin_act_quant_i8(const void* x, int64_t ldx, int64_t M, int64_t K,
                      int8_t* xq, int64_t ldxq, float* xs, void* stream);

/* INT8 x INT8 GEMV with exact int32 accumulation and the epilogue
 *   acc[m,n] = sum_k xq[m,k] * w[n,k]                      (exact, int32)
 *   y[m,n]   = bf16( (fp32(acc) * xs[m]) * ws[n] )          (two fp32 products)
 *   y[m,n]   = bf16( fp32(y[m,n]) + fp32(bias[n]) )         (only if bias != NULL)
 *   xq   int8 [M, ldxq]; xs fp32 [M] (xs_per_token = 1) or [1] (= 0, broadcast)
 *   w    int8 [N, ldw];  ws fp32 [N] (ws_per_row = 1) or [1] (= 0, broadcast)
 *   bias bf16 [N] or NULL
 *   out_kind 0: y is bf16 [M, ldy] holding the epilogue result;
 *   out_kind 1: y is int32 [M, ldy] holding acc (scales and bias unused).
 * Requires K % 16 == 0, 16 <= K <= 131072 (int32 cannot overflow),
 * ldxq % 16 == 0, ldw % 16 == 0, N >= 1, ldy >= N. */
int qlin_gemv_i8(const int8_t* xq, int64_t ldxq, const float* xs, int xs_per_token,
                 int64_t M, int64_t K,
                 const int8_t* w, int64_t ldw, int64_t N,
                 const float* ws, int ws_per_row, const void* bias,
                 void* y, int64_t ldy, int out_kind, void* stream);

/* The whole INT8 decode linear layer in one call: qlin_act_quant_i8 on x
 * (codes and scales written to xq / xs, exactly as that call writes them)
 * followed by qlin_gemv_i8 with out_kind 0 and per-token scales.  For one
 * token (M = 1, K <= 8192) a single kernel does both: each workgroup
 * quantises the row into its LDS (the same fp32 operations, bit-identical
 * codes and outputs) while its weight rows are in flight; otherwise the two
 * kernels run back to back on `stream`.  xq and xs are always written.
 * Arguments, layouts and limits as the two calls ([Z100] section 2.1 times
 * the INT8 GEMV both alone and with its quantiser, the "full" figure). */
int qlin_linear_i8(const void* x, int64_t ldx, int64_t M, int64_t K,
                   const int8_t* w, int64_t ldw, int64_t N, const float* ws, int ws_per_row,
                   const void* bias, int8_t* xq, int64_t ldxq, float* xs,
                   void* y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------
 * (b) FP8-E4M3 weight-only -- [Z100] operator-family table (FP8 row), 2.2
 * ------------------------------------------------------------------------ */

/* y[m,n] = bf16( ws[n] * sum_k e4m3(w[n,k]) * x[m,k] )
 * The weights stay E4M3 in memory and are converted as they are read; the
 * scale is applied once to the fp32 sum.  Accumulation is fp32.
 *   x  bf16 [M, ldx];  w OCP E4M3 codes [N, ldw];
 *   ws fp32 [N] (ws_per_row = 1, per-channel) or [1] (= 0, per-tensor)
 *   y  bf16 [M, ldy]
 * Requires K % 16 == 0, K >= 16, ldx % 8 == 0, ldw % 16 == 0, ldy >= N. */
int qlin_gemv_fp8(const void* x, int64_t ldx, int64_t M, int64_t K,
                  const uint8_t* w, int64_t ldw, int64_t N,
                  const float* ws, int ws_per_row,
                  void* y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------
 * (b') FP8 W8A8 -- [Z100] operator-family table (FP8 row: W8A8 with
 *      e4m3fn or e5m2 codes, per-tensor / per-channel / per-token scales)
 *      and 2.2 (the scale multiplies the accumulated sum once)
 * ------------------------------------------------------------------------ */

/* Dynamic FP8 activation quantisation (the INT8 rule with the format's
 * largest finite value fmax = 448 (E4M3) or 57344 (E5M2) in place of 127):
 *   per_token = 1:  s[m] = max_k |x[m,k]| / fmax,         xs fp32 [M]
 *   per_token = 0:  s    = max_{m,k} |x[m,k]| / fmax,     xs fp32 [1]
 *   xq[m,k] = fp8_rne(x[m,k] / s)   (codes of format fmt, uint8 [M, ldxq])
 * Both divisions are IEEE fp32 (a reciprocal-multiply would change codes);
 * fp8_rne rounds to the nearest finite code, ties to the even code, and a
 * quotient above fmax (a rounding excess) saturates to +-fmax.  A zero
 * amax gives s = 0 and codes 0.  Inputs must be finite.
 * Requires K % 16 == 0, 16 <= K <= 2^24, ldx % 8 == 0, ldxq % 16 == 0,
 * M <= QLIN_MAX_M when per_token = 0 (one workgroup reduces the whole
 * tensor); fmt is QLIN_FMT_E4M3 or QLIN_FMT_E5M2 and per_token 0 or 1 (else
 * QLIN_ERR_ARG). */
int qlin_act_quant_fp8(const void* x, int64_t ldx, int64_t M, int64_t K, int fmt, int per_token,
                       uint8_t* xq, int64_t ldxq, float* xs, void* stream);

/* FP8 x FP8 GEMV:
 *   acc[m,n] = sum_k fp8(xq[m,k]) * fp8(w[n,k])      (fp32 accumulation)
 *   y[m,n]   = bf16( (acc * xs[m]) * ws[n] )          (two fp32 products)
 *   xq codes of format x_fmt [M, ldxq]; xs fp32 [M] (xs_per_token = 1) or
 *   [1] (= 0); w codes of format w_fmt [N, ldw]; ws fp32 [N] (ws_per_row =
 *   1, per-channel) or [1] (= 0, per-tensor); y bf16 [M, ldy].
 * Both operands are widened to bf16 exactly, so each product is exact and
 * only the running fp32 sum rounds.  Weight codes must be finite.
 * Requires K % 16 == 0, 16 <= K <= 2^24, ldxq % 16 == 0, ldw % 16 == 0,
 * N >= 1, ldy >= N; formats and flags as above (else QLIN_ERR_ARG). */
int qlin_gemv_fp8_w8a8(const uint8_t* xq, int64_t ldxq, const float* xs, int xs_per_token, int x_fmt,
                       int64_t M, int64_t K,
                       const uint8_t* w, int64_t ldw, int64_t N,
                       const float* ws, int ws_per_row, int w_fmt,
                       void* y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------
 * (c) Block-scaled FP8 -- [Z100] 2.4 (block formula, scale folding, padded
 *     row stride); [DSV4] 3.3 (dynamic E4M3 activations, UE8M0 scales,
 *     128x128 weight blocks) and 7.4 (UE8M0: scale = 2^(byte - 127))
 * ------------------------------------------------------------------------ */

/* Two steps, one call:
 * 1. Activation quantisation per token m and 128-wide K group kb:
 *      E = 127 + p, p the smallest integer with max|x| <= 448 * 2^p,
 *      clamped to [1, 254] (E = 127 for an all-zero group);
 *      xq[m,k] = e4m3_rne(x[m,k] / 2^(E-127)),  xs[m,kb] = E.
 *    xq / xs are written to the caller's buffers (they are also the exported
 *    quantised activations).  For M = 1 and K <= 32768 both steps run in one
 *    kernel (each workgroup quantises the row into its LDS, and each group is
 *    written to xq / xs by exactly one workgroup); there xq and xs are
 *    optional (NULL: not exported).  Otherwise the step-2 kernel reads xq /
 *    xs back, so both are required (QLIN_ERR_NULL).  The results are the
 *    same either way.  Overflow: an activation group is scaled by a power of
 *    two chosen so that its codes never saturate, but a weight-scale product
 *    (2^(xs-127) * 2^(ws-127) times a block sum) can exceed fp32; such an
 *    output is +-inf or NaN, unspecified, like other non-finite results.
 * 2. out[m,n] = sum_kb ( sum_{k in kb} xq[m,k] * w[n,k] )
 *                     * 2^(xs[m,kb]-127) * 2^(ws[n/128, kb]-127)
 *    The block scales multiply each lane's partial sum of the current block
 *    before any reduction (scale folding), the activation scale first:
 *    (partial * 2^(xs-127)) * 2^(ws-127).  The activation scale follows the
 *    data, so the intermediate stays near the output's own magnitude and an
 *    extreme weight scale byte (0 or 254) cannot overflow or underflow it
 *    first.  fp32 accumulation; y = bf16(out).
 *   x  bf16 [M, ldx]; w E4M3 [N, ldw]; ws UE8M0 [ceil(N/128), K/128]
 *   (row-major, byte 255 decodes to NaN); xq uint8 [M, K]; xs uint8
 *   [M, K/128]; y bf16 [M, ldy].
 * Requires K % 128 == 0, K >= 128, ldx % 8 == 0, ldw % 16 == 0, ldy >= N. */
int qlin_gemv_fp8_blk(const void* x, int64_t ldx, int64_t M, int64_t K,
                      const uint8_t* w, int64_t ldw, int64_t N,
                      const uint8_t* ws,
                      uint8_t* xq, uint8_t* xs,
                      void* y, int64_t ldy, void* stream);

/* The same block-scaled path at any block shape: block_n x block_k weight
 * blocks and block_k-wide activation groups, block_k a multiple of 32 and
 * block_n >= 1 (block_n = 1, block_k = 32 is the MX layout: one UE8M0 scale
 * per row and 32 K elements).  [Z100] 2.4 gives block_n and block_k as
 * run-time parameters with block_k % 32 == 0 (tested there at 128 x 128 only).
 * Arithmetic as qlin_gemv_fp8_blk with 128 replaced by the block sizes:
 *   ws UE8M0 [ceil(N/block_n), K/block_k]; xq uint8 [M, K];
 *   xs uint8 [M, K/block_k]; out[m,n] = sum_kb 2^(xs[m,kb]-127) *
 *   2^(ws[n/block_n,kb]-127) * sum_{k in kb} xq[m,k] * w[n,k].
 * block_n = block_k = 128 is exactly qlin_gemv_fp8_blk.  Other shapes, up to
 * 16 tokens, run a matrix-core GEMV that folds both scales into each block's
 * partial sum.  Above 16 tokens with K % 128 == 0 one tiled GEMM covers all
 * tokens and applies both scales inside the E4M3 -> bf16 operand converts,
 * so the fp32 sum is over exactly scaled products: exact while every scaled
 * value is a normal bf16 number, i.e. weight scale bytes 10..246 and
 * activation groups whose amax exceeds about 2^-109 (the float comparison
 * rule holds either way only inside that range).  Above 16 tokens with
 * K % 128 != 0 the GEMV runs once per 16 tokens (the weights are read once
 * per 16 tokens).  K <= 32768 (the GEMV stages a tile's scale bytes in
 * LDS).  Requires K % block_k == 0, ldx % 8 == 0, ldw % 16 == 0, ldy >= N. */
int qlin_gemv_fp8_blk_ex(const void* x, int64_t ldx, int64_t M, int64_t K,
                         const uint8_t* w, int64_t ldw, int64_t N, const uint8_t* ws,
                         int64_t block_n, int64_t block_k,
                         uint8_t* xq, uint8_t* xs, void* y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------
 * (d) MXFP4 expert GEMV behind top-k routing -- [DSV4] 9.3; element and
 *     scale formats of the OCP MX spec (E2M1, one UE8M0 per 32 elements)
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace qlin_moe_mxfp4 needs for these sizes: the
 * per-(token, slot) fp32 partial rows, M * topk * N * 4 rounded up to 256;
 * for M > 16 followed by the pair sort: int32 pair offsets [E+1], tile
 * offsets [E+1] and pair order [M * topk], rounded up to 256. */
size_t qlin_moe_mxfp4_workspace_bytes(int64_t M, int64_t N, int64_t topk, int64_t E);

/* y[t,n] = bf16( sum_{j < topk} g[t,j] * sum_k e2m1(W[e,n,k]) * 2^(S[e,n,k/32]-127) * x[t,k] ),
 *          e = topk_ids[t,j]
 * Steps: every (token, slot) pair is bucketed by its expert on the device;
 * each live expert's weights are streamed once for all its tokens (fp32
 * partial per pair into the workspace); then the partials are combined in
 * slot order j = 0..topk-1.  No host synchronisation.  For M > 16 (prefill)
 * the pairs are sorted by expert and a grouped matrix-core GEMM computes
 * 64 pairs x 64 rows per workgroup; there the block scale is applied in the
 * E2M1 -> bf16 convert, exact for scale bytes 2..252 (values within bf16's
 * normal range; the M <= 16 path folds the scale in fp32 at any byte).
 *   x         bf16 [M, ldx]
 *   w_fp4     uint8 [E, N, K/2]: element 2i of a row in the LOW nibble of byte i
 *   s_ue8m0   uint8 [E, N, K/32]
 *   topk_ids  int32 [M, topk]: an id outside [0, E) contributes nothing
 *   topk_w    fp32  [M, topk]
 *   y         bf16 [M, ldy]
 *   workspace device buffer of at least qlin_moe_mxfp4_workspace_bytes(),
 *             16-byte aligned; its contents on entry do not matter.
 * Requires K % 32 == 0, 32 <= K <= 30720 (one staged activation row must fit
 * the workgroup's 64 KiB LDS budget), 1 <= topk <= 16, E >= 1, ldx % 8 == 0,
 * M <= QLIN_MAX_M_PREFILL, and E <= 1024 when M > 16. */
int qlin_moe_mxfp4(const void* x, int64_t ldx, int64_t M, int64_t K,
                   const uint8_t* w_fp4, const uint8_t* s_ue8m0, int64_t E, int64_t N,
                   const int32_t* topk_ids, const float* topk_w, int64_t topk,
                   void* y, int64_t ldy,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Largest workspace qlin_moe_mxfp4_noalloc can use (4 MiB): enough for
 * M * topk * N <= 1,048,576 at M <= 16 (M = 16, topk = 8, N = 8192), less
 * the pair-sort arrays above 16 tokens. */
#define QLIN_NOALLOC_SCRATCH_BYTES (4u << 20)

/* qlin_moe_mxfp4 for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * library-owned device array of QLIN_NOALLOC_SCRATCH_BYTES per GPU, held until
 * the process ends.  The caller still passes inputs and outputs.  The call
 * allocates nothing (no hipMalloc/hipFree, no allocating library routine);
 * the first call on a GPU looks up that GPU's copy of the array
 * (hipGetSymbolAddress, the stream's device made current for the lookup).
 * Arguments, layouts and errors as qlin_moe_mxfp4, and QLIN_ERR_WORKSPACE when
 * qlin_moe_mxfp4_workspace_bytes(M, N, topk, E) exceeds
 * QLIN_NOALLOC_SCRATCH_BYTES.  Every call on one GPU shares that GPU's
 * array: two calls that can overlap on one GPU (different streams, or
 * different host threads) race and may give wrong results; serialise them.
 * Nothing in the array needs to start at zero (every value read was written
 * earlier in the same call). */
int qlin_moe_mxfp4_noalloc(const void* x, int64_t ldx, int64_t M, int64_t K,
                           const uint8_t* w_fp4, const uint8_t* s_ue8m0, int64_t E, int64_t N,
                           const int32_t* topk_ids, const float* topk_w, int64_t topk,
                           void* y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------
 * (e) Routed MXFP4 expert FFN with on-device routing -- [DSV4] 9.3 (MXFP4
 *     expert path), 6.6 (J09) and 9.4 (SwiGLU: alpha 1.0, limit 10.0),
 *     0.1/0.2 (the routing fast path stays on the device)
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace qlin_moe_ffn_mxfp4 needs for these sizes: the
 * router logits fp32 [M][E], then the SwiGLU activations bf16 [M*topk][I],
 * then the down-projection partials fp32 [M*topk][H], each region starting
 * on a 256-byte boundary (in that order, from the workspace base). */
size_t qlin_moe_ffn_mxfp4_workspace_bytes(int64_t M, int64_t H, int64_t I, int64_t topk, int64_t E);

/* For every token t (x row, H = hidden size):
 *   logit[t,e] = sum_k x[t,k] * wr[e,k]            (bf16 router, fp32 sum)
 *   ids[t,:]   = the topk largest logits, largest first; equal logits go to
 *                the lower expert id; a NaN logit ranks as -inf
 *   g[t,j]     = exp(logit[t,ids[t,j]] - logit[t,ids[t,0]]) / sum over the
 *                topk selected (softmax over the selected logits)
 *   for each slot j, e = ids[t,j], i < I:
 *     gate_i = w13[e, i, :] . x[t],  up_i = w13[e, I+i, :] . x[t]   (MXFP4)
 *     act[t*topk+j, i] = bf16( silu(alpha * min(gate_i, limit))
 *                              * clamp(up_i, -limit, limit) ),  silu(z) = z/(1+e^-z)
 *   y[t,h] = bf16( sum_j g[t,j] * (w2[e, h, :] . act[t*topk+j]) )   (slot order)
 * MXFP4 rows are E2M1 codes (element 2i in the LOW nibble of byte i) with
 * one UE8M0 scale per 32 elements; every dot accumulates in fp32.  Five
 * kernels on `stream`, no host synchronisation.
 *   x        bf16 [M, ldx]
 *   wr       bf16 [E, H] (row-major)
 *   w13      uint8 [E, 2I, H/2]: gate rows 0..I-1, then up rows I..2I-1
 *   s13      uint8 [E, 2I, H/32]
 *   w2       uint8 [E, H, I/2];  s2 uint8 [E, H, I/32]
 *   topk_ids int32 [M, topk] (output);  topk_w fp32 [M, topk] (output)
 *   y        bf16 [M, ldy]
 *   workspace device buffer of at least qlin_moe_ffn_mxfp4_workspace_bytes(),
 *            16-byte aligned; contents on entry do not matter, on return it
 *            holds the logits and activations described there.
 * Requires 1 <= M <= 16, 1 <= E <= 1024, 1 <= topk <= min(16, E),
 * H and I multiples of 32 in [32, 30720], ldx >= H with ldx % 8 == 0,
 * ldy >= H. */
int qlin_moe_ffn_mxfp4(const void* x, int64_t ldx, int64_t M, int64_t H,
                       const void* wr, int64_t E, int64_t topk,
                       const uint8_t* w13, const uint8_t* s13, int64_t I,
                       const uint8_t* w2, const uint8_t* s2,
                       float alpha, float limit,
                       int32_t* topk_ids, float* topk_w,
                       void* y, int64_t ldy,
                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
