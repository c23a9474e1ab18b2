/*
 * zq.h -- C ABI of libzq, the fused quantized linear layer of ZeroQuant
 * (arXiv 2206.01861) as hand-written HIP kernels for MI355X (gfx950).
 *
 * Source pages: "ZeroQuant: Efficient and Affordable Post-Training
 * Quantization for Large-Scale Transformers", long-form summary
 * (paper-graph-ui), Sec. 3.4 "Group-wise Weight Quantization" (paper
 * Sec. 4.1, Eq. (2)), "Token-wise Activation Quantization" (paper Sec. 4.1)
 * and "Quantization-Optimized Transformer Kernels" (paper Sec. 4.3, App. D,
 * Fig. 2).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    compute calls never allocate, free or synchronize; each enqueues its
 *    kernels on `stream` (a hipStream_t; NULL means the null stream) and
 *    returns at once.  Results are ready when the stream reaches them.
 *    (The schedule tuner synchronizes, and a chain owns host memory, one
 *    HIP stream and its graphs; both are described where declared.)
 *  - All matrices are row-major and dense.  Activations are [M][K] (one
 *    row per token = batch*seqlen entry), weights [N][K] (one row per output
 *    feature, K contiguous), outputs [M][N].
 *  - fp16 means IEEE binary16.  Scales are fp32.
 *  - Arguments are checked before anything is launched.  A failed check
 *    returns a non-zero zq_status and launches nothing; the reason is kept
 *    in a thread-local string returned by zq_last_error().  M == 0 is a
 *    valid empty call (ZQ_OK, nothing launched); buffers sized by M may
 *    then be NULL.
 *  - Alignment (PyTorch allocations satisfy all of it): GEMM operands (qx,
 *    qw, qw4, the fp16 x of zq_gemm_w8a16), int32 outputs, quantized
 *    outputs qy and workspaces 16 bytes; GEMM outputs y 8
 *    bytes; fp32 arrays 4 bytes; other fp16 tensors (x of the quantizers,
 *    gamma, beta, bias, ln_out) 2 bytes.  A misaligned pointer returns
 *    ZQ_EINVAL.  fp16 tensors that are not 16-byte aligned take slower
 *    element-wise loads; the results are the same.
 *  - Calls on one stream run in order; calls on different streams that
 *    write the same memory race, as with any kernel.
 */
#ifndef ZQ_H
#define ZQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ZQ_OK = 0,
    ZQ_EINVAL = 1,       /* null or misaligned pointer, bad bits or act   */
    ZQ_ESHAPE = 2,       /* negative/zero sizes, N % G != 0, odd K for W4 */
    ZQ_EHIP = 3,         /* the HIP runtime refused a launch              */
    ZQ_EUNSUPPORTED = 4  /* valid but outside the implemented range       */
} zq_status;

typedef enum { ZQ_ACT_NONE = 0, ZQ_ACT_GELU = 1 } zq_act;

/* Largest K accepted by zq_ln_quant_act / zq_quant_act (a token row is held
 * in registers).  Larger K returns ZQ_EUNSUPPORTED. */
#define ZQ_MAX_ROW_K 65536
/* Largest K accepted by the GEMMs.  The calls take any two's-complement
 * code, including -128 (int8) and -8 (nibble), which Eq. (2)'s integer
 * range [-2^(b-1), 2^(b-1) - 1] admits although the quantizer never emits
 * them.  The largest product magnitude is then 128 * 128 = 16384 for W8,
 * and 16 * 8 * 128 = 16384 for the W4 path, which accumulates 16 * acc;
 * K * 16384 <= 2^31 - 1 holds up to K = 131071, and the largest multiple
 * of 64 below that is 131008. */
#define ZQ_MAX_GEMM_K_W8 131008
#define ZQ_MAX_GEMM_K_W4 131008

/*
 * zq_quantize_weights -- group-wise symmetric weight quantization
 * (Sec. 3.4 "Group-wise Weight Quantization", paper Sec. 4.1, Eq. (2)).
 *
 * W[N][K] fp16 is split into N/G groups of G contiguous rows (output
 * features).  Group g has scale S_g = max|W[gG:(g+1)G, :]| / qmax with
 * qmax = 127 (bits = 8) or 7 (bits = 4), and codes
 *     q = rint(clamp(W / S_g, -qmax, qmax))   (fp32 IEEE division,
 *                                              round half to even)
 * An all-zero group gets S_g = 0 and zero codes.
 *   bits = 8: qw is int8 [N][K].
 *   bits = 4: qw is uint8 [N][K/2]; byte j of a row holds k = 2j in its low
 *             nibble and k = 2j+1 in its high nibble, two's complement.
 *   sw: fp32 [N/G].
 * Errors: ZQ_EINVAL (null pointer, bits not 4/8), ZQ_ESHAPE (N, K or G <= 0,
 * N % G != 0, odd K with bits = 4).  One workgroup per group; an offline
 * step, not on the per-token path.
 */
zq_status zq_quantize_weights(const void *w_fp16, int N, int K, int G,
                              int bits, void *qw, float *sw, void *stream);

/*
 * zq_ln_quant_act -- LayerNorm fused with dynamic token-wise INT8
 * quantization (Sec. 3.4 "Quantization-Optimized Transformer Kernels",
 * paper App. D, Fig. 2; token-wise scale from "Token-wise Activation
 * Quantization", paper Sec. 4.1).
 *
 * Per token row t of x fp16 [M][K]:
 *     mean, biased variance over K (fp32),
 *     h = fp16((x - mean) / sqrt(var + eps) * gamma + beta),
 *     sx[t] = max_k |h| / 127,
 *     qx[t][k] = rint(clamp(h / sx[t], -127, 127))   (0 if sx[t] == 0).
 * Only int8 codes and one fp32 scale per token leave the kernel; h stays in
 * registers unless ln_out is given.
 *   gamma, beta: fp16 [K], each may be NULL (1 and 0).
 *   qx: int8 [M][K]; sx: fp32 [M]; ln_out: fp16 [M][K] or NULL.
 * Errors: ZQ_EINVAL (null x/qx/sx), ZQ_ESHAPE (M < 0, K <= 0),
 * ZQ_EUNSUPPORTED (K > ZQ_MAX_ROW_K).
 */
zq_status zq_ln_quant_act(const void *x_fp16, const void *gamma_fp16,
                          const void *beta_fp16, float eps, int M, int K,
                          int8_t *qx, float *sx, void *ln_out_fp16,
                          void *stream);

/*
 * zq_quant_act -- token-wise INT8 quantization without LayerNorm, for the
 * GEMM inputs that follow a bias-add or GeLU rather than a LayerNorm
 * (Sec. 3.4 "Quantization-Optimized Transformer Kernels", paper App. D).
 * Same quantizer as zq_ln_quant_act applied to x itself.
 *   x: fp16 [M][K]; qx: int8 [M][K]; sx: fp32 [M].
 * Errors as zq_ln_quant_act.
 */
zq_status zq_quant_act(const void *x_fp16, int M, int K, int8_t *qx,
                       float *sx, void *stream);

/*
 * zq_gemm_w8a8 -- INT8 x INT8 GEMM with the dequantization fused into the
 * epilogue (Sec. 3.4 "Quantization-Optimized Transformer Kernels", paper
 * Sec. 4.3 and App. D):
 *     acc[t][n] = sum_k qx[t][k] * qw[n][k]           (exact, int32)
 *     y[t][n]   = fp16(act(acc * (sx[t] * sw[n / G]) + bias[n]))
 * act: ZQ_ACT_NONE or ZQ_ACT_GELU (exact erf form).  The fp32 epilogue is
 * computed in registers; only fp16 y is written.
 *   qx int8 [M][K], sx fp32 [M], qw int8 [N][K], sw fp32 [N/G],
 *   bias fp16 [N] or NULL, y fp16 [M][N].
 * Errors: ZQ_EINVAL (null/misaligned pointer, act not 0/1), ZQ_ESHAPE
 * (M < 0, N or K <= 0, G <= 0, N % G != 0), ZQ_EUNSUPPORTED (K % 64 != 0,
 * K > ZQ_MAX_GEMM_K_W8).
 */
zq_status zq_gemm_w8a8(const int8_t *qx, const float *sx, const int8_t *qw,
                       const float *sw, int G, const void *bias_fp16, int act,
                       int M, int N, int K, void *y_fp16, void *stream);

/*
 * zq_gemm_w4a8 -- as zq_gemm_w8a8 with nibble-packed INT4 weights (the
 * mixed W4/8 scheme puts INT4 on the feed-forward weights, Sec. 3.4
 * "Group-wise Weight Quantization", paper Sec. 5).  qw4 is uint8 [N][K/2]
 * in the zq_quantize_weights(bits = 4) layout; nibbles are expanded to int8
 * in registers and fed to the same INT8 matrix instructions.
 * Errors as zq_gemm_w8a8, with K limited to ZQ_MAX_GEMM_K_W4.
 */
zq_status zq_gemm_w4a8(const int8_t *qx, const float *sx, const uint8_t *qw4,
                       const float *sw, int G, const void *bias_fp16, int act,
                       int M, int N, int K, void *y_fp16, void *stream);

/*
 * zq_gemm_w8a8_i32 / zq_gemm_w4a8_i32 -- the same main loops with a raw
 * epilogue: acc int32 [M][N] = sum_k qx[t][k] * qw[n][k].  These expose the
 * integer accumulator (paper App. D: the INT32 result before
 * dequantization) so that it can be compared exactly.
 * Errors as the fused calls (no G/bias/act arguments).
 */
zq_status zq_gemm_w8a8_i32(const int8_t *qx, const int8_t *qw, int M, int N,
                           int K, int32_t *acc, void *stream);
zq_status zq_gemm_w4a8_i32(const int8_t *qx, const uint8_t *qw4, int M, int N,
                           int K, int32_t *acc, void *stream);

/*
 * zq_gemm_w8a8_quant / zq_gemm_w4a8_quant -- the GEMM with its output
 * quantized token-wise for the next linear (the inputs of attn-out and
 * FFN2 follow a bias-add or GeLU, and the token quantization is fused into
 * that producing step: Sec. 3.4 "Quantization-Optimized Transformer
 * Kernels", paper App. D).  Arguments as zq_gemm_w8a8 / _w4a8, but instead
 * of y the call writes
 *   qy int8 [M][N] and sy fp32 [M]  (16- and 4-byte aligned)
 * equal, bit for bit, to zq_gemm_w8a8 (fp16 y) followed by zq_quant_act(y):
 * sy[t] = max_n |y[t][n]| / 127 over the fp16 outputs, qy = the codes.
 * The fp16 output is written to the workspace and quantized from there
 * (two kernels on the stream).  A token's scale needs all N outputs of its
 * row, which different workgroups produce; quantizing inside the GEMM
 * epilogue would need a device-wide barrier, which costs more on this GPU
 * than the fp16 round trip it saves.
 *   ws: device workspace of at least zq_gemm_quant_workspace_bytes(M, N)
 *       (= 2 M N) bytes, 16-byte aligned, owned by the caller; clobbered.
 *       Calls that share a workspace must be ordered (same stream).
 * Errors as zq_gemm_w8a8, plus ZQ_EINVAL for a null or short workspace or
 * null qy/sy, and ZQ_EUNSUPPORTED for N > ZQ_MAX_ROW_K.
 */
zq_status zq_gemm_w8a8_quant(const int8_t *qx, const float *sx,
                             const int8_t *qw, const float *sw, int G,
                             const void *bias_fp16, int act, int M, int N,
                             int K, int8_t *qy, float *sy, void *ws,
                             size_t ws_bytes, void *stream);
zq_status zq_gemm_w4a8_quant(const int8_t *qx, const float *sx,
                             const uint8_t *qw4, const float *sw, int G,
                             const void *bias_fp16, int act, int M, int N,
                             int K, int8_t *qy, float *sy, void *ws,
                             size_t ws_bytes, void *stream);
/* Workspace bytes the _quant calls need for an M x N output (0 if M or N
 * is not positive). */
size_t zq_gemm_quant_workspace_bytes(int M, int N);

/*
 * zq_gemm_w8a8_xq / zq_gemm_w4a8_xq -- the linear of an fp16 activation
 * with its token-wise quantization done by the consuming GEMM (the fused
 * quantization in front of attn-out and FFN2 of Sec. 3.4
 * "Quantization-Optimized Transformer Kernels", paper App. D, Fig. 2,
 * taken on the consumer's side).  The result is bit for bit that of
 * zq_quant_act(x) -> (qx, sx) followed by zq_gemm_w8a8 / _w4a8 on
 * (qx, sx):
 *   x   fp16 [M][K] (device, 16-byte aligned): e.g. the fp16 y of the
 *       previous linear's zq_gemm_w8a8 with its bias and GeLU
 *   qx  int8 [M][K], sx fp32 [M] (device, caller-owned, 16- and 4-byte
 *       aligned): receive the codes and scales
 *   y   fp16 [M][N]; qw/qw4, sw, G, bias, act, M, N, K as zq_gemm_w8a8.
 * One token (M == 1) where zq_gemm_plan is the GEMV with the activation
 * row in LDS (K <= 32768): one kernel.  Every block loads the whole fp16
 * row, takes its max |x| and quantizes it into LDS, so no block needs
 * another's result, and the quantizer launch with its fp16 read and code
 * write disappear (block 0 writes qx and sx for the caller).  Elsewhere
 * the row quantizer runs first and the plan's kernel reads qx and sx: at
 * many tokens each workgroup of the consumer would have to quantize the
 * activation tiles it shares with the others again, which costs more than
 * the launch it saves.  zq_gemm_xq_plan says which form runs.
 * Errors: as zq_gemm_w8a8, ZQ_EINVAL for a null or misaligned x/qx/sx, and
 * ZQ_EUNSUPPORTED for K > ZQ_MAX_ROW_K.
 */
zq_status zq_gemm_w8a8_xq(const void *x_fp16, const int8_t *qw, const float *sw,
                          int G, const void *bias_fp16, int act, int M, int N,
                          int K, void *y_fp16, int8_t *qx, float *sx,
                          void *stream);
zq_status zq_gemm_w4a8_xq(const void *x_fp16, const uint8_t *qw4,
                          const float *sw, int G, const void *bias_fp16,
                          int act, int M, int N, int K, void *y_fp16,
                          int8_t *qx, float *sx, void *stream);
zq_status zq_gemm_xq_plan(int M, int N, int K, int bits, char *buf,
                          int buflen);

/*
 * zq_gemm_w8a8_ws / zq_gemm_w4a8_ws -- zq_gemm_w8a8 / zq_gemm_w4a8 with a
 * caller workspace, for decode-sized token counts over few weight tiles
 * (the small-batch schedules of the summary page's Sec. 3.4
 * "Quantization-Optimized Transformer Kernels", paper App. D: at small
 * batch the GEMM is bound by weight bandwidth, and every compute unit must
 * stream).  For 33 .. 64 tokens where 64 x 64 tiles would leave compute
 * units idle (packed W4: when K splits into at least 4 slices), K is split
 * over several workgroups per tile: each writes
 * exact int32 partial sums into the workspace, and a second kernel adds
 * them and applies the same epilogue, so y is bit-identical to the call
 * without a workspace.  Other shapes run exactly as that call.
 *   ws: device memory of at least zq_gemm_workspace_bytes(M, N, K, bits)
 *   bytes, 16-byte aligned, owned by the caller; its contents on entry do
 *   not matter and are overwritten (two calls sharing one workspace on
 *   different streams race).  When that size is 0, ws may be NULL.
 * A schedule-table entry for the shape takes precedence (no split).
 * Errors: as zq_gemm_w8a8; ZQ_EINVAL (workspace NULL, misaligned or
 * smaller than needed).
 * zq_gemm_workspace_bytes: the bytes these calls need for the shape (0
 * when they would not split; also 0 for invalid arguments).
 * zq_gemm_ws_plan: the plan these calls run, as zq_gemm_plan.
 */
zq_status zq_gemm_w8a8_ws(const int8_t *qx, const float *sx, const int8_t *qw,
                          const float *sw, int G, const void *bias_fp16,
                          int act, int M, int N, int K, void *y_fp16, void *ws,
                          size_t ws_bytes, void *stream);
zq_status zq_gemm_w4a8_ws(const int8_t *qx, const float *sx, const uint8_t *qw4,
                          const float *sw, int G, const void *bias_fp16,
                          int act, int M, int N, int K, void *y_fp16, void *ws,
                          size_t ws_bytes, void *stream);
size_t zq_gemm_workspace_bytes(int M, int N, int K, int bits);
zq_status zq_gemm_ws_plan(int M, int N, int K, int bits, char *buf, int buflen);

/*
 * zq_gemm_noalloc -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): zq_gemm_w8a8_ws (bits = 8) or zq_gemm_w4a8_ws (bits = 4)
 * with the split-K partial sums in a scratch array that the library holds
 * in device memory, ZQ_NOALLOC_SCRATCH_BYTES per device, from the first
 * call on that device until the process ends, instead of a caller
 * workspace.  No allocation happens in the call.  y is bit-identical to the
 * _ws call's.
 *   Arguments as zq_gemm_w8a8 / zq_gemm_w4a8 (qw: int8 [N][K] or packed
 *   uint8 [N][K/2]), plus bits.
 * Every call on one GPU shares that GPU's scratch array: calls that overlap
 * on one GPU (different streams, or threads without ordering) race, and the
 * array keeps the last call's contents (nothing in it needs to start at
 * zero: each split writes its whole partial plane before it is read).
 * Errors: as zq_gemm_w8a8; ZQ_EINVAL (bits not 4 or 8); ZQ_EUNSUPPORTED if
 * the split would need more than ZQ_NOALLOC_SCRATCH_BYTES (the built-in
 * splits need at most that: 33..64 tokens over fewer than 128 64x64 tiles,
 * SK slices x M x N x 4 bytes <= 4 MiB) or the device index is 64 or more;
 * ZQ_EHIP if the scratch array has no device address.
 */
#define ZQ_NOALLOC_SCRATCH_BYTES (4u << 20)
zq_status zq_gemm_noalloc(int bits, const int8_t *qx, const float *sx,
                          const void *qw, const float *sw, int G,
                          const void *bias_fp16, int act, int M, int N, int K,
                          void *y_fp16, void *stream);

/*
 * zq_calibrate_minmax / zq_quant_act_static -- static per-tensor activation
 * quantization, the prior-PTQ scheme that token-wise scales replace
 * (summary page Sec. 3.4 "Token-wise Activation Quantization"; paper
 * App. B.1), kept as a comparator.
 * zq_calibrate_minmax: one calibration batch x fp16 [M][K] moves the device
 * state fp32 [2] = {x_min, x_max}:  first != 0 sets it to the batch's min
 * and max; otherwise x = momentum * x + (1 - momentum) * batch value, fp32
 * with each product and the sum rounded once (the pages use momentum 0.95).
 * One workgroup (an offline step).
 * zq_quant_act_static: Eq. (2) over the whole tensor with the frozen scale
 * S = max(|x_min|, |x_max|) / 127 read from the device state; values beyond
 * the range clamp to +-127.  qx int8 [M][K]; s_out fp32 [1] receives S.
 * Errors: ZQ_EINVAL (null/misaligned pointer, momentum outside [0, 1]),
 * ZQ_ESHAPE (M < 0 (calibration: M <= 0), K <= 0).
 */
zq_status zq_calibrate_minmax(const void *x_fp16, int M, int K, float momentum,
                              int first, float *state, void *stream);
zq_status zq_quant_act_static(const void *x_fp16, int M, int K,
                              const float *state, int8_t *qx, float *s_out,
                              void *stream);

/*
 * zq_gemm_w8a16 -- INT8 group-wise weights with FP16 activations, the mixed
 * scheme of the summary page's Sec. 5 "Experimental Analysis" (Table 4: W8A16;
 * Table 8: GPT-NeoX20B keeps its self-attention inputs in FP16 while the
 * weights are INT8):
 *     y[t][n] = fp16(act(sw[n / G] * sum_k x[t][k] * qw[n][k] + bias[n]))
 * The codes enter an fp16 matrix multiply unchanged (every INT8 value is
 * exact in fp16) with fp32 accumulation; the group scale, constant along k,
 * is applied in the epilogue, so no dequantized weight is ever rounded.
 *   x fp16 [M][K] (16-byte aligned), qw int8 [N][K], sw fp32 [N/G],
 *   bias fp16 [N] or NULL, y fp16 [M][N].
 * Errors: ZQ_EINVAL (null/misaligned pointer, act not 0/1), ZQ_ESHAPE
 * (M < 0, N or K <= 0, G <= 0, N % G != 0), ZQ_EUNSUPPORTED (K % 64 != 0,
 * K > ZQ_MAX_GEMM_K_A16).
 */
#define ZQ_MAX_GEMM_K_A16 1048576
zq_status zq_gemm_w8a16(const void *x_fp16, const int8_t *qw, const float *sw,
                        int G, const void *bias_fp16, int act, int M, int N,
                        int K, void *y_fp16, void *stream);
/* The tile configuration zq_gemm_w8a16 picks (as zq_gemm_plan). */
zq_status zq_gemm_w8a16_plan(int M, int N, int K, char *buf, int buflen);

/*
 * Chunk-contiguous weights for decode -- the codes of zq_quantize_weights in
 * another order, for the weight-streaming GEMM at 1 .. 16 tokens, where the
 * linear is bound by reading its weights from HBM (the small-batch
 * schedules of the summary page's Sec. 3.4 "Quantization-Optimized
 * Transformer Kernels", paper App. D).  Values and scales are unchanged;
 * the bytes of each chunk of BN rows x CK row bytes are stored as one
 * contiguous range, chunks in order along the row and row blocks in order
 * along N:
 *     qd[((rb * (R / CK) + c) * BN + r) * CK + b] = qw[(rb * BN + r) * R + c * CK + b]
 * with R = K (W8) or K / 2 (W4, the packed bytes as they are), so the
 * kernel's copies read 1 KB of consecutive bytes where the row-major layout
 * gives 1024 / CK rows at a row stride.  BN and CK are fixed per shape
 * (zq_chunked_layout; the same on every device).  The buffer has the size
 * of the row-major one.
 *
 * zq_chunked_layout: the rows per block (16 or 32) and chunk bytes (128,
 *   256 or 512) of the shape.
 * zq_pack_chunked: row-major codes qw (int8 [N][K], or packed uint8
 *   [N][K/2]) -> qd.  An offline step, asynchronous on stream; qw and qd
 *   must not overlap.
 * zq_gemm_w8a8_chunked / zq_gemm_w4a8_chunked: zq_gemm_w8a8 / zq_gemm_w4a8
 *   with the weights in this layout, for 0 <= M <= 16 tokens (M = 0
 *   writes nothing); y is bit-identical to those calls on the row-major
 *   codes.  The bias, when given, must be 4-byte aligned; act as for
 *   zq_gemm_w8a8.
 * zq_gemm_chunked_i32: the raw int32 accumulator (test hook), bits 8 or 4.
 * zq_gemm_chunked_plan: the kernel configuration for the shape.
 * Errors: ZQ_EINVAL (null/misaligned pointer as for zq_gemm_w8a8, a bias
 * not 4-byte aligned, act not 0 or 1, bits not 4 or 8, overlapping
 * qw / qd), ZQ_ESHAPE
 * (M < 0, N or K <= 0, G <= 0, N % G != 0), ZQ_EUNSUPPORTED (K % 64 != 0,
 * N not a multiple of BN or the row bytes not a multiple of CK, K above
 * ZQ_MAX_GEMM_K_W8 / _W4, M > 16).
 */
zq_status zq_chunked_layout(int N, int K, int bits, int *rows,
                            int *chunk_bytes);
zq_status zq_pack_chunked(const void *qw, int N, int K, int bits, void *qd,
                          void *stream);
zq_status zq_gemm_w8a8_chunked(const int8_t *qx, const float *sx,
                               const int8_t *qd, const float *sw, int G,
                               const void *bias_fp16, int act, int M, int N,
                               int K, void *y_fp16, void *stream);
zq_status zq_gemm_w4a8_chunked(const int8_t *qx, const float *sx,
                               const uint8_t *qd4, const float *sw, int G,
                               const void *bias_fp16, int act, int M, int N,
                               int K, void *y_fp16, void *stream);
zq_status zq_gemm_chunked_i32(int bits, const int8_t *qx, const void *qd,
                              int M, int N, int K, int32_t *acc, void *stream);
zq_status zq_gemm_chunked_plan(int M, int N, int K, int bits, char *buf,
                               int buflen);

/*
 * zq_gemm_plan -- which kernel and tile shape the GEMM calls pick for a
 * problem (the schedule chosen by token count, paper App. D), written as a
 * NUL-terminated string into buf (at most buflen bytes).  No launch.
 * Errors: ZQ_EINVAL (null buf, buflen <= 0), as zq_gemm_w8a8 for shapes.
 */
zq_status zq_gemm_plan(int M, int N, int K, int bits, char *buf, int buflen);

/*
 * Schedule table -- the pages profile several GEMM schedules (tilings) for
 * each input-size combination and, at run time, use the one profiled for
 * the current batch x seqlen (summary page Sec. 3.4 "Quantization-Optimized
 * Transformer Kernels", the schedule profiling and small-batch paragraphs;
 * paper Sec. 4.3, App. D).  Here a process-wide table maps (bits, N, K,
 * M range) to a kernel and tile; zq_gemm_w8a8/w4a8 (and their _i32 and
 * _quant forms) and zq_gemm_plan consult it before the built-in rules.
 * A plan never changes results: every kernel and tile gives the same bits.
 * The table is shared by all threads and devices of the process (guarded
 * by a lock); an empty table gives the built-in rules.
 *
 * zq_gemm_tune: times every kernel and tile that applies at each token
 * count ms[0 .. nm-1] (strictly ascending, >= 1) for the problem described
 * by the arguments (the same as zq_gemm_w8a8, bits 8 or 4, on buffers
 * sized for M = ms[nm-1]; y is overwritten), `reps` launches each after
 * one warm-up, and stores the fastest for the token range (ms[i-1], ms[i]]
 * (ms[-1] = 0).  chosen (nm x 2 ints: kind 0 skinny, 1 tiled, 2 stream,
 * 3 gemv; tile index or -1) and us (nm floats, the winner's average
 * launch time in microseconds) may be NULL.  Synchronizes `stream`; must
 * not be called while `stream` is being captured.  The split over K of the
 * workspace calls (zq_gemm_w8a8_ws) is not among the timed plans; a table
 * entry for a shape turns that split off.
 * Errors: as zq_gemm_w8a8; ZQ_EINVAL (ms not ascending or < 1, nm < 1 or
 * > 64, reps < 1 or > 10000, stream under capture).
 *
 * zq_sched_export: the table as text, one entry per line:
 *     "<bits> <N> <K> <M lo> <M hi> <skinny|tiled|stream|gemv> <tile>"
 * written NUL-terminated into buf (truncated to buflen - 1 chars; buf may
 * be NULL with buflen 0); *needed (may be NULL) receives the full size
 * including the NUL.  zq_sched_import: adds the entries of such a text
 * (blank lines and '#' comments are skipped), replacing what the table
 * holds for the same (bits, N, K) over each range; either every line is
 * valid and all are added, or nothing is (ZQ_EINVAL, the first bad line
 * named in zq_last_error).  A kernel must apply at both ends of its range
 * (gemv: M = 1 with whole 1 KB weight-row pieces; stream: M <= 16, even N;
 * skinny: M <= 64; tile indices of W8-only tiles are refused for bits 4).
 * zq_sched_clear empties the table.  zq_sched_entries: entry count.
 */
zq_status zq_gemm_tune(int bits, const int8_t *qx, const float *sx,
                       const void *qw, const float *sw, int G,
                       const void *bias_fp16, int act, const int *ms, int nm,
                       int N, int K, void *y_fp16, int reps, int *chosen,
                       float *us, void *stream);
zq_status zq_sched_export(char *buf, size_t buflen, size_t *needed);
zq_status zq_sched_import(const char *text);
void zq_sched_clear(void);
int zq_sched_entries(void);

/*
 * zq_chain -- a recorded sequence of the calls above, replayed as one HIP
 * graph: the pages record a small model's whole launch sequence on the
 * first inference call and replay it with a single submission afterwards,
 * removing per-kernel launch overhead (summary page Sec. 3.4
 * "Quantization-Optimized Transformer Kernels", the CUDA Graph paragraph;
 * paper App. D).
 *
 * zq_chain_create(max_m): an empty chain whose buffers hold up to max_m
 * token rows.  The zq_chain_add_* calls append one call each, with the
 * arguments of the call of the same name minus M and stream; every buffer
 * sized by M must hold max_m rows (row r of each begins at the same offset
 * as in a dense [max_m][...] tensor) and stays owned by the caller, who
 * keeps it allocated while the chain lives.  Arguments are checked when
 * added, as the call itself checks them (with M = max_m; ws_bytes against
 * the largest workspace any token count up to max_m needs), and a failing
 * add appends nothing.  Host only: no GPU is touched.  zq_chain_add_gemm_ws
 * records zq_gemm_w8a8_ws (bits 8) or zq_gemm_w4a8_ws (bits 4), and
 * zq_chain_add_gemm_xq zq_gemm_w8a8_xq or zq_gemm_w4a8_xq (the graph for
 * one token holds its single kernel, the graphs for more tokens the
 * quantizer and the GEMM).  zq_chain_add_gemm_chunked records
 * zq_gemm_w8a8_chunked or zq_gemm_w4a8_chunked (weights in the chunked
 * decode layout; the chain's max_m must be at most 16, else
 * ZQ_EUNSUPPORTED).
 *
 * zq_chain_run(chain, M, stream): runs the sequence over the first M rows
 * of every buffer.  The first run with a given M (or the first after the
 * schedule table changed) captures the launches into a HIP graph on a
 * stream of the chain's own (created then, on the current device, which
 * must hold the buffers) and instantiates it; every run launches the
 * graph for its M on `stream`.  If `stream` is itself being captured, the
 * calls are launched directly instead, so they join that capture.  At most
 * ZQ_CHAIN_MAX_GRAPHS graphs are kept (the least recently used is dropped).
 * zq_chain_run_eager launches the same calls one by one, without a graph.
 * M == 0 launches nothing.  The graphs read the buffers' contents at each
 * launch, so new inputs need no new capture.  A chain is used by one
 * thread at a time; runs on different streams that share buffers race.
 * zq_chain_graphs: graphs currently held; zq_chain_length: calls recorded.
 * zq_chain_destroy frees the graphs, the stream and the chain (NULL is
 * ignored).  Freeing a graph that was ever launched (on destruction, when
 * the cache drops one, or when the schedule table changed) first waits for
 * the whole device (hipDeviceSynchronize), since its launches went to the
 * callers' streams; runs themselves add nothing to the stream.
 * Errors: ZQ_EINVAL (null chain, max_m < 1, M outside [0, max_m]), the
 * add errors of the matching call, ZQ_EHIP (capture or launch refused).
 */
typedef struct zq_chain zq_chain;
#define ZQ_CHAIN_MAX_GRAPHS 64
zq_status zq_chain_create(int max_m, zq_chain **out);
zq_status zq_chain_add_ln_quant(zq_chain *c, const void *x_fp16,
                                const void *gamma_fp16, const void *beta_fp16,
                                float eps, int K, int8_t *qx, float *sx,
                                void *ln_out_fp16);
zq_status zq_chain_add_quant(zq_chain *c, const void *x_fp16, int K,
                             int8_t *qx, float *sx);
zq_status zq_chain_add_gemm(zq_chain *c, int bits, const int8_t *qx,
                            const float *sx, const void *qw, const float *sw,
                            int G, const void *bias_fp16, int act, int N, int K,
                            void *y_fp16);
zq_status zq_chain_add_gemm_quant(zq_chain *c, int bits, const int8_t *qx,
                                  const float *sx, const void *qw,
                                  const float *sw, int G, const void *bias_fp16,
                                  int act, int N, int K, int8_t *qy, float *sy,
                                  void *ws, size_t ws_bytes);
zq_status zq_chain_add_gemm_ws(zq_chain *c, int bits, const int8_t *qx,
                               const float *sx, const void *qw, const float *sw,
                               int G, const void *bias_fp16, int act, int N,
                               int K, void *y_fp16, void *ws, size_t ws_bytes);
zq_status zq_chain_add_gemm_w8a16(zq_chain *c, const void *x_fp16,
                                  const int8_t *qw, const float *sw, int G,
                                  const void *bias_fp16, int act, int N, int K,
                                  void *y_fp16);
zq_status zq_chain_add_gemm_chunked(zq_chain *c, int bits, const int8_t *qx,
                                    const float *sx, const void *qd,
                                    const float *sw, int G,
                                    const void *bias_fp16, int act, int N,
                                    int K, void *y_fp16);
zq_status zq_chain_add_gemm_xq(zq_chain *c, int bits, const void *x_fp16,
                               const void *qw, const float *sw, int G,
                               const void *bias_fp16, int act, int N, int K,
                               void *y_fp16, int8_t *qx, float *sx);
zq_status zq_chain_run(zq_chain *c, int M, void *stream);
zq_status zq_chain_run_eager(zq_chain *c, int M, void *stream);
int zq_chain_graphs(const zq_chain *c);
int zq_chain_length(const zq_chain *c);
void zq_chain_destroy(zq_chain *c);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char *zq_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int zq_version(void);
#define ZQ_VERSION 106

#ifdef __cplusplus
}
#endif

#endif /* ZQ_H */
