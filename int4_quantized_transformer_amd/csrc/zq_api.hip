// zq_api.hip -- the extern "C" entry points declared in include/zq.h:
// argument checks, error reporting and dispatch to the kernels.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "zq_internal.h"

namespace zq {

static thread_local char g_err[512] = "";

zq_status fail(zq_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

zq_status ok() {
  g_err[0] = '\0';
  return ZQ_OK;
}

}  // namespace zq

namespace {

using zq::fail;
using zq::ok;

zq_status hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess)
    return fail(ZQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Buffers sized by M (qx, sx, y, acc) may be NULL when M == 0.
zq_status check_gemm(const int8_t *qx, const void *qw, int M, int N, int K,
                     int bits, const char *fn) {
  if ((!qx && M != 0) || !qw) return fail(ZQ_EINVAL, "%s: null qx/qw", fn);
  if (!aligned(qx, 16) || !aligned(qw, 16))
    return fail(ZQ_EINVAL, "%s: qx/qw must be 16-byte aligned", fn);
  if (M < 0 || N <= 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape M=%d N=%d K=%d", fn, M, N, K);
  if (K % 64 != 0)
    return fail(ZQ_EUNSUPPORTED, "%s: K=%d is not a multiple of 64", fn, K);
  const int kmax = bits == 4 ? ZQ_MAX_GEMM_K_W4 : ZQ_MAX_GEMM_K_W8;
  if (K > kmax)
    return fail(ZQ_EUNSUPPORTED,
                "%s: K=%d exceeds %d (int32 accumulator bound)", fn, K, kmax);
  return ZQ_OK;
}

zq_status gemm_fused(const int8_t *qx, const float *sx, const void *qw,
                     const float *sw, int G, const void *bias, int act, int M,
                     int N, int K, void *y, void *stream, int bits,
                     const char *fn) {
  zq_status st = check_gemm(qx, qw, M, N, K, bits, fn);
  if (st != ZQ_OK) return st;
  if (!sw || ((!sx || !y) && M != 0))
    return fail(ZQ_EINVAL, "%s: null sx/sw/y", fn);
  if (!aligned(sx, 4) || !aligned(sw, 4) || !aligned(y, 8) ||
      (bias && !aligned(bias, 2)))
    return fail(ZQ_EINVAL, "%s: misaligned sx/sw/y/bias", fn);
  if (act != ZQ_ACT_NONE && act != ZQ_ACT_GELU)
    return fail(ZQ_EINVAL, "%s: act=%d", fn, act);
  if (G <= 0 || N % G != 0)
    return fail(ZQ_ESHAPE, "%s: N=%d is not a multiple of G=%d", fn, N, G);
  if (M == 0) return ok();
  zq::GemmArgs a{};
  a.qx = qx;
  a.sx = sx;
  a.qw = qw;
  a.sw = sw;
  a.bias = static_cast<const zq::half_t *>(bias);
  a.out = y;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.act = act;
  a.bits = bits;
  a.raw_i32 = false;
  return hip_status(zq::launch_gemm(a, (hipStream_t)stream), fn);
}

zq_status gemm_with_ws(const int8_t *qx, const float *sx, const void *qw,
                       const float *sw, int G, const void *bias, int act,
                       int M, int N, int K, void *y, void *ws,
                       size_t ws_bytes, void *stream, int bits,
                       const char *fn) {
  zq_status st = check_gemm(qx, qw, M, N, K, bits, fn);
  if (st != ZQ_OK) return st;
  if (!sw || ((!sx || !y) && M != 0))
    return fail(ZQ_EINVAL, "%s: null sx/sw/y", fn);
  if (!aligned(sx, 4) || !aligned(sw, 4) || !aligned(y, 8) ||
      !aligned(ws, 16) || (bias && !aligned(bias, 2)))
    return fail(ZQ_EINVAL, "%s: misaligned sx/sw/y/ws/bias", fn);
  if (act != ZQ_ACT_NONE && act != ZQ_ACT_GELU)
    return fail(ZQ_EINVAL, "%s: act=%d", fn, act);
  if (G <= 0 || N % G != 0)
    return fail(ZQ_ESHAPE, "%s: N=%d is not a multiple of G=%d", fn, N, G);
  if (M == 0) return ok();
  const size_t need = zq::gemm_ws_bytes(M, N, K, bits);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(ZQ_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn,
                ws ? ws_bytes : 0, need);
  zq::GemmArgs a{};
  a.qx = qx;
  a.sx = sx;
  a.qw = qw;
  a.sw = sw;
  a.bias = static_cast<const zq::half_t *>(bias);
  a.out = y;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.act = act;
  a.bits = bits;
  a.raw_i32 = false;
  return hip_status(zq::launch_gemm_ws(a, need > 0 ? ws : nullptr,
                                       (hipStream_t)stream),
                    fn);
}

zq_status gemm_quant_out(const int8_t *qx, const float *sx, const void *qw,
                         const float *sw, int G, const void *bias, int act,
                         int M, int N, int K, int8_t *qy, float *sy, void *ws,
                         size_t ws_bytes, void *stream, int bits,
                         const char *fn) {
  zq_status st = check_gemm(qx, qw, M, N, K, bits, fn);
  if (st != ZQ_OK) return st;
  if (!sw || ((!sx || !qy || !sy || !ws) && M != 0))
    return fail(ZQ_EINVAL, "%s: null sx/sw/qy/sy/ws", fn);
  if (!aligned(sx, 4) || !aligned(sw, 4) || !aligned(sy, 4) ||
      !aligned(qy, 16) || !aligned(ws, 16) || (bias && !aligned(bias, 2)))
    return fail(ZQ_EINVAL, "%s: misaligned sx/sw/sy/qy/ws/bias", fn);
  if (act != ZQ_ACT_NONE && act != ZQ_ACT_GELU)
    return fail(ZQ_EINVAL, "%s: act=%d", fn, act);
  if (G <= 0 || N % G != 0)
    return fail(ZQ_ESHAPE, "%s: N=%d is not a multiple of G=%d", fn, N, G);
  if (N > ZQ_MAX_ROW_K)
    return fail(ZQ_EUNSUPPORTED, "%s: N=%d exceeds %d", fn, N, ZQ_MAX_ROW_K);
  if (M == 0) return ok();
  const size_t need = zq::gemm_quant_ws_bytes(M, N);
  if (ws_bytes < need)
    return fail(ZQ_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn,
                ws_bytes, need);
  zq::GemmArgs a{};
  a.qx = qx;
  a.sx = sx;
  a.qw = qw;
  a.sw = sw;
  a.bias = static_cast<const zq::half_t *>(bias);
  a.out = nullptr;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.act = act;
  a.bits = bits;
  a.raw_i32 = false;
  return hip_status(zq::launch_gemm_quant(a, qy, sy, ws, (hipStream_t)stream),
                    fn);
}

zq_status gemm_xq(const void *x, const void *qw, const float *sw, int G,
                  const void *bias, int act, int M, int N, int K, void *y,
                  int8_t *qx, float *sx, void *stream, int bits,
                  const char *fn) {
  zq_status st = check_gemm(qx, qw, M, N, K, bits, fn);
  if (st != ZQ_OK) return st;
  if (!sw || ((!x || !sx || !y) && M != 0))
    return fail(ZQ_EINVAL, "%s: null x/sx/sw/y", fn);
  if (!aligned(x, 16) || !aligned(sx, 4) || !aligned(sw, 4) ||
      !aligned(y, 8) || (bias && !aligned(bias, 2)))
    return fail(ZQ_EINVAL, "%s: misaligned x/sx/sw/y/bias", fn);
  if (act != ZQ_ACT_NONE && act != ZQ_ACT_GELU)
    return fail(ZQ_EINVAL, "%s: act=%d", fn, act);
  if (G <= 0 || N % G != 0)
    return fail(ZQ_ESHAPE, "%s: N=%d is not a multiple of G=%d", fn, N, G);
  if (K > ZQ_MAX_ROW_K)
    return fail(ZQ_EUNSUPPORTED, "%s: K=%d exceeds %d", fn, K, ZQ_MAX_ROW_K);
  if (M == 0) return ok();
  zq::GemmArgs a{};
  a.qx = static_cast<const int8_t *>(x);  // fp16 bytes
  a.sx = nullptr;
  a.qw = qw;
  a.sw = sw;
  a.bias = static_cast<const zq::half_t *>(bias);
  a.out = y;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.act = act;
  a.bits = bits;
  a.raw_i32 = false;
  return hip_status(zq::launch_gemm_xq(a, qx, sx, (hipStream_t)stream), fn);
}

zq_status gemm_raw(const int8_t *qx, const void *qw, int M, int N, int K,
                   int32_t *acc, void *stream, int bits, const char *fn) {
  zq_status st = check_gemm(qx, qw, M, N, K, bits, fn);
  if (st != ZQ_OK) return st;
  if (!acc && M != 0) return fail(ZQ_EINVAL, "%s: null acc", fn);
  if (!aligned(acc, 16)) return fail(ZQ_EINVAL, "%s: acc must be 16-byte aligned", fn);
  if (M == 0) return ok();
  zq::GemmArgs a{};
  a.qx = qx;
  a.qw = qw;
  a.out = acc;
  a.G = 1;
  a.M = M;
  a.N = N;
  a.K = K;
  a.bits = bits;
  a.raw_i32 = true;
  return hip_status(zq::launch_gemm(a, (hipStream_t)stream), fn);
}

zq_status row_quant(const void *x, const void *gamma, const void *beta,
                    float eps, int M, int K, bool ln, int8_t *qx, float *sx,
                    void *ln_out, void *stream, const char *fn) {
  if ((!x || !qx || !sx) && M != 0)
    return fail(ZQ_EINVAL, "%s: null x/qx/sx", fn);
  if (!aligned(x, 2) || !aligned(sx, 4) || (gamma && !aligned(gamma, 2)) ||
      (beta && !aligned(beta, 2)) || (ln_out && !aligned(ln_out, 2)))
    return fail(ZQ_EINVAL, "%s: misaligned pointer", fn);
  if (M < 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape M=%d K=%d", fn, M, K);
  if (K > ZQ_MAX_ROW_K)
    return fail(ZQ_EUNSUPPORTED, "%s: K=%d exceeds %d", fn, K, ZQ_MAX_ROW_K);
  if (ln && !(eps >= 0.0f))
    return fail(ZQ_EINVAL, "%s: eps must be >= 0", fn);
  if (M == 0) return ok();
  return hip_status(zq::launch_row_quant(x, gamma, beta, eps, M, K, ln, qx,
                                         sx, ln_out, (hipStream_t)stream),
                    fn);
}

// Shapes of the chunk-contiguous weight layout: the 16-token ring's row
// blocks and chunks must tile the matrix.
zq_status check_chunked_shape(int N, int K, int bits, const char *fn) {
  if (bits != 8 && bits != 4) return fail(ZQ_EINVAL, "%s: bits=%d", fn, bits);
  if (N <= 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape N=%d K=%d", fn, N, K);
  if (K % 64 != 0)
    return fail(ZQ_EUNSUPPORTED, "%s: K=%d is not a multiple of 64", fn, K);
  int bn = 0, ck = 0;
  if (!zq::chunked_layout(N, K, bits, &bn, &ck, nullptr))
    return fail(ZQ_EUNSUPPORTED,
                "%s: N=%d K=%d W%d does not tile into %d-row blocks of "
                "%d-byte chunks", fn, N, K, bits, bn, ck);
  return ZQ_OK;
}

zq_status gemm_chunked(const int8_t *qx, const float *sx, const void *qd,
                       const float *sw, int G, const void *bias, int act,
                       int M, int N, int K, void *out, bool raw, void *stream,
                       int bits, const char *fn) {
  zq_status st = check_chunked_shape(N, K, bits, fn);
  if (st != ZQ_OK) return st;
  st = check_gemm(qx, qd, M, N, K, bits, fn);
  if (st != ZQ_OK) return st;
  if (M > 16)
    return fail(ZQ_EUNSUPPORTED, "%s: M=%d exceeds 16 tokens", fn, M);
  if (!out && M != 0) return fail(ZQ_EINVAL, "%s: null output", fn);
  if (raw) {
    if (!aligned(out, 16))
      return fail(ZQ_EINVAL, "%s: acc must be 16-byte aligned", fn);
  } else {
    if (!sw || (!sx && M != 0)) return fail(ZQ_EINVAL, "%s: null sx/sw", fn);
    // the ring gathers the bias as pairs of columns (4-byte words)
    if (!aligned(sx, 4) || !aligned(sw, 4) || !aligned(out, 8) ||
        (bias && !aligned(bias, 4)))
      return fail(ZQ_EINVAL, "%s: misaligned sx/sw/y/bias (bias: 4 bytes)",
                  fn);
    if (act != ZQ_ACT_NONE && act != ZQ_ACT_GELU)
      return fail(ZQ_EINVAL, "%s: act=%d", fn, act);
    if (G <= 0 || N % G != 0)
      return fail(ZQ_ESHAPE, "%s: N=%d is not a multiple of G=%d", fn, N, G);
  }
  if (M == 0) return ok();
  zq::GemmArgs a{};
  a.qx = qx;
  a.sx = raw ? nullptr : sx;
  a.qw = qd;
  a.sw = raw ? nullptr : sw;
  a.bias = raw ? nullptr : static_cast<const zq::half_t *>(bias);
  a.out = out;
  a.G = raw ? 1 : G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.act = raw ? 0 : act;
  a.bits = bits;
  a.raw_i32 = raw;
  return hip_status(zq::launch_gemm_chunked(a, (hipStream_t)stream), fn);
}

// ------------------------------------------------- device-resident scratch
// The split-K workspace of zq_gemm_noalloc: one array per device, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address; its device address is looked up once per device (with
// that device current) and only that address is passed to kernels.
static __device__ __align__(256) char scratch[ZQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices] = {};

static zq_status scratch_for_current_device(void **out, const char *fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ZQ_EUNSUPPORTED, "%s: device %d beyond the %d supported", fn,
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ZQ_EHIP, "%s: no device address for the scratch array: %s",
                  fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ZQ_OK;
}

}  // namespace

extern "C" {

zq_status zq_quantize_weights(const void *w_fp16, int N, int K, int G,
                              int bits, void *qw, float *sw, void *stream) {
  const char *fn = "zq_quantize_weights";
  if (!w_fp16 || !qw || !sw) return fail(ZQ_EINVAL, "%s: null pointer", fn);
  if (bits != 8 && bits != 4) return fail(ZQ_EINVAL, "%s: bits=%d", fn, bits);
  if (!aligned(w_fp16, 2) || !aligned(sw, 4))
    return fail(ZQ_EINVAL, "%s: misaligned pointer", fn);
  if (N <= 0 || K <= 0 || G <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape N=%d K=%d G=%d", fn, N, K, G);
  if (N % G != 0)
    return fail(ZQ_ESHAPE, "%s: N=%d is not a multiple of G=%d", fn, N, G);
  if (bits == 4 && K % 2 != 0)
    return fail(ZQ_ESHAPE, "%s: W4 needs an even K (K=%d)", fn, K);
  return hip_status(zq::launch_quantize_weights(w_fp16, N, K, G, bits, qw, sw,
                                                (hipStream_t)stream),
                    fn);
}

zq_status zq_ln_quant_act(const void *x_fp16, const void *gamma_fp16,
                          const void *beta_fp16, float eps, int M, int K,
                          int8_t *qx, float *sx, void *ln_out_fp16,
                          void *stream) {
  return row_quant(x_fp16, gamma_fp16, beta_fp16, eps, M, K, true, qx, sx,
                   ln_out_fp16, stream, "zq_ln_quant_act");
}

zq_status zq_quant_act(const void *x_fp16, int M, int K, int8_t *qx,
                       float *sx, void *stream) {
  return row_quant(x_fp16, nullptr, nullptr, 0.0f, M, K, false, qx, sx,
                   nullptr, stream, "zq_quant_act");
}

zq_status zq_gemm_w8a8(const int8_t *qx, const float *sx, const int8_t *qw,
                       const float *sw, int G, const void *bias_fp16, int act,
                       int M, int N, int K, void *y_fp16, void *stream) {
  return gemm_fused(qx, sx, qw, sw, G, bias_fp16, act, M, N, K, y_fp16,
                    stream, 8, "zq_gemm_w8a8");
}

zq_status zq_gemm_w4a8(const int8_t *qx, const float *sx, const uint8_t *qw4,
                       const float *sw, int G, const void *bias_fp16, int act,
                       int M, int N, int K, void *y_fp16, void *stream) {
  return gemm_fused(qx, sx, qw4, sw, G, bias_fp16, act, M, N, K, y_fp16,
                    stream, 4, "zq_gemm_w4a8");
}

zq_status zq_gemm_w8a8_i32(const int8_t *qx, const int8_t *qw, int M, int N,
                           int K, int32_t *acc, void *stream) {
  return gemm_raw(qx, qw, M, N, K, acc, stream, 8, "zq_gemm_w8a8_i32");
}

zq_status zq_gemm_w4a8_i32(const int8_t *qx, const uint8_t *qw4, int M, int N,
                           int K, int32_t *acc, void *stream) {
  return gemm_raw(qx, qw4, M, N, K, acc, stream, 4, "zq_gemm_w4a8_i32");
}

zq_status zq_gemm_w8a8_quant(const int8_t *qx, const float *sx,
                             const int8_t *qw, const float *sw, int G,
                             const void *bias_fp16, int act, int M, int N,
                             int K, int8_t *qy, float *sy, void *ws,
                             size_t ws_bytes, void *stream) {
  return gemm_quant_out(qx, sx, qw, sw, G, bias_fp16, act, M, N, K, qy, sy, ws,
                        ws_bytes, stream, 8, "zq_gemm_w8a8_quant");
}

zq_status zq_gemm_w4a8_quant(const int8_t *qx, const float *sx,
                             const uint8_t *qw4, const float *sw, int G,
                             const void *bias_fp16, int act, int M, int N,
                             int K, int8_t *qy, float *sy, void *ws,
                             size_t ws_bytes, void *stream) {
  return gemm_quant_out(qx, sx, qw4, sw, G, bias_fp16, act, M, N, K, qy, sy,
                        ws, ws_bytes, stream, 4, "zq_gemm_w4a8_quant");
}

zq_status zq_gemm_w8a8_xq(const void *x_fp16, const int8_t *qw, const float *sw,
                          int G, const void *bias_fp16, int act, int M, int N,
                          int K, void *y_fp16, int8_t *qx, float *sx,
                          void *stream) {
  return gemm_xq(x_fp16, qw, sw, G, bias_fp16, act, M, N, K, y_fp16, qx, sx,
                 stream, 8, "zq_gemm_w8a8_xq");
}

zq_status zq_gemm_w4a8_xq(const void *x_fp16, const uint8_t *qw4,
                          const float *sw, int G, const void *bias_fp16,
                          int act, int M, int N, int K, void *y_fp16,
                          int8_t *qx, float *sx, void *stream) {
  return gemm_xq(x_fp16, qw4, sw, G, bias_fp16, act, M, N, K, y_fp16, qx, sx,
                 stream, 4, "zq_gemm_w4a8_xq");
}

zq_status zq_gemm_xq_plan(int M, int N, int K, int bits, char *buf,
                          int buflen) {
  const char *fn = "zq_gemm_xq_plan";
  if (!buf || buflen <= 0) return fail(ZQ_EINVAL, "%s: null buffer", fn);
  if (bits != 8 && bits != 4) return fail(ZQ_EINVAL, "%s: bits=%d", fn, bits);
  if (M < 0 || N <= 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape M=%d N=%d K=%d", fn, M, N, K);
  zq::describe_gemm_xq_plan(M, N, K, bits, buf, buflen);
  return ok();
}

zq_status zq_gemm_w8a8_ws(const int8_t *qx, const float *sx, const int8_t *qw,
                          const float *sw, int G, const void *bias_fp16,
                          int act, int M, int N, int K, void *y_fp16, void *ws,
                          size_t ws_bytes, void *stream) {
  return gemm_with_ws(qx, sx, qw, sw, G, bias_fp16, act, M, N, K, y_fp16, ws,
                      ws_bytes, stream, 8, "zq_gemm_w8a8_ws");
}

zq_status zq_gemm_w4a8_ws(const int8_t *qx, const float *sx, const uint8_t *qw4,
                          const float *sw, int G, const void *bias_fp16,
                          int act, int M, int N, int K, void *y_fp16, void *ws,
                          size_t ws_bytes, void *stream) {
  return gemm_with_ws(qx, sx, qw4, sw, G, bias_fp16, act, M, N, K, y_fp16, ws,
                      ws_bytes, stream, 4, "zq_gemm_w4a8_ws");
}

zq_status zq_gemm_noalloc(int bits, const int8_t *qx, const float *sx,
                          const void *qw, const float *sw, int G,
                          const void *bias_fp16, int act, int M, int N, int K,
                          void *y_fp16, void *stream) {
  const char *fn = "zq_gemm_noalloc";
  if (bits != 8 && bits != 4) return fail(ZQ_EINVAL, "%s: bits=%d", fn, bits);
  zq_status st = check_gemm(qx, qw, M, N, K, bits, fn);
  if (st != ZQ_OK) return st;
  if (!sw || ((!sx || !y_fp16) && M != 0))
    return fail(ZQ_EINVAL, "%s: null sx/sw/y", fn);
  if (!aligned(sx, 4) || !aligned(sw, 4) || !aligned(y_fp16, 8) ||
      (bias_fp16 && !aligned(bias_fp16, 2)))
    return fail(ZQ_EINVAL, "%s: misaligned sx/sw/y/bias", fn);
  if (act != ZQ_ACT_NONE && act != ZQ_ACT_GELU)
    return fail(ZQ_EINVAL, "%s: act=%d", fn, act);
  if (G <= 0 || N % G != 0)
    return fail(ZQ_ESHAPE, "%s: N=%d is not a multiple of G=%d", fn, N, G);
  if (M == 0) return ok();
  const size_t need = zq::gemm_ws_bytes(M, N, K, bits);
  if (need > ZQ_NOALLOC_SCRATCH_BYTES)
    return fail(ZQ_EUNSUPPORTED,
                "%s: the split needs %zu bytes of scratch, more than the %u "
                "the library holds per device",
                fn, need, (unsigned)ZQ_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (need > 0) {
    st = scratch_for_current_device(&ws, fn);
    if (st != ZQ_OK) return st;
  }
  zq::GemmArgs a{};
  a.qx = qx;
  a.sx = sx;
  a.qw = qw;
  a.sw = sw;
  a.bias = static_cast<const zq::half_t *>(bias_fp16);
  a.out = y_fp16;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.act = act;
  a.bits = bits;
  a.raw_i32 = false;
  return hip_status(zq::launch_gemm_ws(a, ws, (hipStream_t)stream), fn);
}

size_t zq_gemm_workspace_bytes(int M, int N, int K, int bits) {
  if (M <= 0 || N <= 0 || K <= 0 || (bits != 8 && bits != 4)) return 0;
  return zq::gemm_ws_bytes(M, N, K, bits);
}

zq_status zq_gemm_ws_plan(int M, int N, int K, int bits, char *buf, int buflen) {
  const char *fn = "zq_gemm_ws_plan";
  if (!buf || buflen <= 0) return fail(ZQ_EINVAL, "%s: null buffer", fn);
  if (bits != 8 && bits != 4) return fail(ZQ_EINVAL, "%s: bits=%d", fn, bits);
  if (M < 0 || N <= 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape M=%d N=%d K=%d", fn, M, N, K);
  zq::describe_gemm_ws_plan(M, N, K, bits, buf, buflen);
  return ok();
}

size_t zq_gemm_quant_workspace_bytes(int M, int N) {
  if (M <= 0 || N <= 0) return 0;
  return zq::gemm_quant_ws_bytes(M, N);
}

zq_status zq_calibrate_minmax(const void *x_fp16, int M, int K, float momentum,
                              int first, float *state, void *stream) {
  const char *fn = "zq_calibrate_minmax";
  if (!state || (!x_fp16 && M != 0)) return fail(ZQ_EINVAL, "%s: null x/state", fn);
  if (!aligned(x_fp16, 2) || !aligned(state, 4))
    return fail(ZQ_EINVAL, "%s: misaligned pointer", fn);
  if (M <= 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape M=%d K=%d", fn, M, K);
  if (!(momentum >= 0.0f && momentum <= 1.0f))
    return fail(ZQ_EINVAL, "%s: momentum must be in [0, 1]", fn);
  return hip_status(zq::launch_calibrate(x_fp16, (size_t)M * K, momentum,
                                         first ? 1 : 0, state,
                                         (hipStream_t)stream),
                    fn);
}

zq_status zq_quant_act_static(const void *x_fp16, int M, int K,
                              const float *state, int8_t *qx, float *s_out,
                              void *stream) {
  const char *fn = "zq_quant_act_static";
  if (!state || !s_out || ((!x_fp16 || !qx) && M != 0))
    return fail(ZQ_EINVAL, "%s: null x/state/qx/s_out", fn);
  if (!aligned(x_fp16, 2) || !aligned(state, 4) || !aligned(s_out, 4))
    return fail(ZQ_EINVAL, "%s: misaligned pointer", fn);
  if (M < 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape M=%d K=%d", fn, M, K);
  if (M == 0) return ok();
  return hip_status(zq::launch_static_quant(x_fp16, (size_t)M * K, state, qx,
                                            s_out, (hipStream_t)stream),
                    fn);
}

zq_status zq_gemm_w8a16(const void *x_fp16, const int8_t *qw, const float *sw,
                        int G, const void *bias_fp16, int act, int M, int N,
                        int K, void *y_fp16, void *stream) {
  const char *fn = "zq_gemm_w8a16";
  if ((!x_fp16 && M != 0) || !qw || !sw || (!y_fp16 && M != 0))
    return fail(ZQ_EINVAL, "%s: null x/qw/sw/y", fn);
  if (!aligned(x_fp16, 16) || !aligned(qw, 16) || !aligned(sw, 4) ||
      !aligned(y_fp16, 8) || (bias_fp16 && !aligned(bias_fp16, 2)))
    return fail(ZQ_EINVAL, "%s: misaligned x/qw/sw/y/bias", fn);
  if (M < 0 || N <= 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape M=%d N=%d K=%d", fn, M, N, K);
  if (act != ZQ_ACT_NONE && act != ZQ_ACT_GELU)
    return fail(ZQ_EINVAL, "%s: act=%d", fn, act);
  if (G <= 0 || N % G != 0)
    return fail(ZQ_ESHAPE, "%s: N=%d is not a multiple of G=%d", fn, N, G);
  if (K % 64 != 0)
    return fail(ZQ_EUNSUPPORTED, "%s: K=%d is not a multiple of 64", fn, K);
  if (K > ZQ_MAX_GEMM_K_A16)
    return fail(ZQ_EUNSUPPORTED, "%s: K=%d exceeds %d", fn, K, ZQ_MAX_GEMM_K_A16);
  if (M == 0) return ok();
  zq::GemmArgs a{};
  a.qx = static_cast<const int8_t *>(x_fp16);  // fp16 bytes
  a.sx = nullptr;
  a.qw = qw;
  a.sw = sw;
  a.bias = static_cast<const zq::half_t *>(bias_fp16);
  a.out = y_fp16;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.act = act;
  a.bits = 8;
  a.raw_i32 = false;
  return hip_status(zq::launch_gemm_w8a16(a, (hipStream_t)stream), fn);
}

zq_status zq_chunked_layout(int N, int K, int bits, int *rows,
                            int *chunk_bytes) {
  const char *fn = "zq_chunked_layout";
  zq_status st = check_chunked_shape(N, K, bits, fn);
  if (st != ZQ_OK) return st;
  zq::chunked_layout(N, K, bits, rows, chunk_bytes, nullptr);
  return ok();
}

zq_status zq_pack_chunked(const void *qw, int N, int K, int bits, void *qd,
                          void *stream) {
  const char *fn = "zq_pack_chunked";
  zq_status st = check_chunked_shape(N, K, bits, fn);
  if (st != ZQ_OK) return st;
  if (!qw || !qd) return fail(ZQ_EINVAL, "%s: null qw/qd", fn);
  if (!aligned(qw, 16) || !aligned(qd, 16))
    return fail(ZQ_EINVAL, "%s: qw/qd must be 16-byte aligned", fn);
  const size_t bytes = (size_t)N * K * bits / 8;
  const char *a = static_cast<const char *>(qw);
  const char *b = static_cast<const char *>(qd);
  if (a < b + bytes && b < a + bytes)
    return fail(ZQ_EINVAL, "%s: qw and qd overlap", fn);
  return hip_status(
      zq::launch_pack_chunked(qw, N, K, bits, qd, (hipStream_t)stream), fn);
}

zq_status zq_gemm_w8a8_chunked(const int8_t *qx, const float *sx,
                               const int8_t *qd, const float *sw, int G,
                               const void *bias_fp16, int act, int M, int N,
                               int K, void *y_fp16, void *stream) {
  return gemm_chunked(qx, sx, qd, sw, G, bias_fp16, act, M, N, K, y_fp16,
                      false, stream, 8, "zq_gemm_w8a8_chunked");
}

zq_status zq_gemm_w4a8_chunked(const int8_t *qx, const float *sx,
                               const uint8_t *qd4, const float *sw, int G,
                               const void *bias_fp16, int act, int M, int N,
                               int K, void *y_fp16, void *stream) {
  return gemm_chunked(qx, sx, qd4, sw, G, bias_fp16, act, M, N, K, y_fp16,
                      false, stream, 4, "zq_gemm_w4a8_chunked");
}

zq_status zq_gemm_chunked_i32(int bits, const int8_t *qx, const void *qd,
                              int M, int N, int K, int32_t *acc,
                              void *stream) {
  const char *fn = "zq_gemm_chunked_i32";
  if (bits != 8 && bits != 4) return fail(ZQ_EINVAL, "%s: bits=%d", fn, bits);
  return gemm_chunked(qx, nullptr, qd, nullptr, 1, nullptr, 0, M, N, K, acc,
                      true, stream, bits, fn);
}

zq_status zq_gemm_chunked_plan(int M, int N, int K, int bits, char *buf,
                               int buflen) {
  const char *fn = "zq_gemm_chunked_plan";
  if (!buf || buflen <= 0) return fail(ZQ_EINVAL, "%s: null buffer", fn);
  zq_status st = check_chunked_shape(N, K, bits, fn);
  if (st != ZQ_OK) return st;
  if (M < 0 || M > 16)
    return fail(ZQ_ESHAPE, "%s: M=%d outside 0..16", fn, M);
  zq::describe_gemm_chunked_plan(M, N, K, bits, buf, buflen);
  return ok();
}

zq_status zq_gemm_w8a16_plan(int M, int N, int K, char *buf, int buflen) {
  const char *fn = "zq_gemm_w8a16_plan";
  if (!buf || buflen <= 0) return fail(ZQ_EINVAL, "%s: null buffer", fn);
  if (M < 0 || N <= 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape M=%d N=%d K=%d", fn, M, N, K);
  zq::describe_gemm_w8a16_plan(M, N, K, buf, buflen);
  return ok();
}

zq_status zq_gemm_plan(int M, int N, int K, int bits, char *buf, int buflen) {
  const char *fn = "zq_gemm_plan";
  if (!buf || buflen <= 0) return fail(ZQ_EINVAL, "%s: null buffer", fn);
  if (bits != 8 && bits != 4) return fail(ZQ_EINVAL, "%s: bits=%d", fn, bits);
  if (M < 0 || N <= 0 || K <= 0)
    return fail(ZQ_ESHAPE, "%s: bad shape M=%d N=%d K=%d", fn, M, N, K);
  zq::describe_gemm_plan(M, N, K, bits, buf, buflen);
  return ok();
}

zq_status zq_gemm_tune(int bits, const int8_t *qx, const float *sx,
                       const void *qw, const float *sw, int G,
                       const void *bias_fp16, int act, const int *ms, int nm,
                       int N, int K, void *y_fp16, int reps, int *chosen,
                       float *us, void *stream) {
  const char *fn = "zq_gemm_tune";
  if (bits != 8 && bits != 4) return fail(ZQ_EINVAL, "%s: bits=%d", fn, bits);
  if (!ms || nm < 1 || nm > 64)
    return fail(ZQ_EINVAL, "%s: need 1 .. 64 token counts (nm=%d)", fn, nm);
  for (int i = 0; i < nm; ++i)
    if (ms[i] < 1 || (i > 0 && ms[i] <= ms[i - 1]))
      return fail(ZQ_EINVAL, "%s: token counts must be >= 1 and ascending", fn);
  if (reps < 1 || reps > 10000)
    return fail(ZQ_EINVAL, "%s: reps=%d outside [1, 10000]", fn, reps);
  if (!qx || !sx || !y_fp16) return fail(ZQ_EINVAL, "%s: null qx/sx/y", fn);
  // the remaining checks of the GEMM call itself (with no launch)
  zq_status st = gemm_fused(qx, sx, qw, sw, G, bias_fp16, act, 0, N, K,
                            y_fp16, stream, bits, fn);
  if (st != ZQ_OK) return st;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  st = hip_status(hipStreamIsCapturing((hipStream_t)stream, &cs), fn);
  if (st != ZQ_OK) return st;
  if (cs != hipStreamCaptureStatusNone)
    return fail(ZQ_EINVAL, "%s: the stream is being captured", fn);
  zq::GemmArgs a{};
  a.qx = qx;
  a.sx = sx;
  a.qw = qw;
  a.sw = sw;
  a.bias = static_cast<const zq::half_t *>(bias_fp16);
  a.out = y_fp16;
  a.G = G;
  a.N = N;
  a.K = K;
  a.act = act;
  a.bits = bits;
  a.raw_i32 = false;
  int kinds[64], cfgs[64];
  st = hip_status(zq::tune_gemm(a, ms, nm, reps, (hipStream_t)stream, kinds,
                                cfgs, us),
                  fn);
  if (st != ZQ_OK) return st;
  if (chosen)
    for (int i = 0; i < nm; ++i) {
      chosen[2 * i] = kinds[i];
      chosen[2 * i + 1] = cfgs[i];
    }
  return ok();
}

zq_status zq_sched_export(char *buf, size_t buflen, size_t *needed) {
  if (!buf && buflen > 0)
    return fail(ZQ_EINVAL, "zq_sched_export: null buffer with buflen > 0");
  const size_t n = zq::sched_export(buf, buflen);
  if (needed) *needed = n;
  return ok();
}

zq_status zq_sched_import(const char *text) {
  if (!text) return fail(ZQ_EINVAL, "zq_sched_import: null text");
  const int r = zq::sched_import(text);
  if (r < 0)
    return fail(ZQ_EINVAL, "zq_sched_import: line %d is not a valid entry", -r);
  return ok();
}

void zq_sched_clear(void) { zq::sched_clear(); }

int zq_sched_entries(void) { return zq::sched_entries(); }

const char *zq_last_error(void) { return zq::g_err; }

int zq_version(void) { return ZQ_VERSION; }

}  // extern "C"
