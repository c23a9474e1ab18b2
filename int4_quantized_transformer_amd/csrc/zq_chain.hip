// zq_chain.hip -- a recorded sequence of libzq calls replayed as HIP graphs.
//
// The pages record a small model's whole launch sequence on the first
// inference call and replay it with one submission afterwards, which takes
// the per-kernel launch cost off the critical path ("ZeroQuant" summary
// page, Sec. 3.4 "Quantization-Optimized Transformer Kernels", the CUDA Graph
// paragraph; paper App. D).  A chain holds the calls with their buffers
// (sized for max_m token rows); a run over M rows launches the graph
// captured for that M, capturing it first if there is none yet or if the
// schedule table changed since (its plans are baked into the graph).
#include <stdint.h>

#include <vector>

#include "zq_internal.h"

namespace {

enum OpKind {
  kLnQuant, kQuant, kGemm, kGemmQuant, kGemmA16, kGemmWs, kGemmXq, kGemmChunked
};

struct ChainOp {
  OpKind kind;
  // row quantizers
  const void *x = nullptr, *gamma = nullptr, *beta = nullptr;
  float eps = 0.0f;
  int8_t *qx = nullptr;
  float *sx = nullptr;
  void *ln_out = nullptr;
  // GEMMs
  int bits = 8;
  const int8_t *gqx = nullptr;
  const float *gsx = nullptr;
  const void *qw = nullptr;
  const float *sw = nullptr;
  int G = 0;
  const void *bias = nullptr;
  int act = 0, N = 0, K = 0;
  void *y = nullptr;
  int8_t *qy = nullptr;
  float *sy = nullptr;
  void *ws = nullptr;
  size_t ws_bytes = 0;
};

struct GraphEntry {
  int M;
  unsigned gen;
  hipGraphExec_t exec;
  bool launched;
  uint64_t last_use;
};

zq_status run_op(const ChainOp &o, int M, void *s) {
  switch (o.kind) {
    case kLnQuant:
      return zq_ln_quant_act(o.x, o.gamma, o.beta, o.eps, M, o.K, o.qx, o.sx,
                             o.ln_out, s);
    case kQuant:
      return zq_quant_act(o.x, M, o.K, o.qx, o.sx, s);
    case kGemm:
      return o.bits == 8
                 ? zq_gemm_w8a8(o.gqx, o.gsx, (const int8_t *)o.qw, o.sw, o.G,
                                o.bias, o.act, M, o.N, o.K, o.y, s)
                 : zq_gemm_w4a8(o.gqx, o.gsx, (const uint8_t *)o.qw, o.sw, o.G,
                                o.bias, o.act, M, o.N, o.K, o.y, s);
    case kGemmQuant:
      return o.bits == 8
                 ? zq_gemm_w8a8_quant(o.gqx, o.gsx, (const int8_t *)o.qw, o.sw,
                                      o.G, o.bias, o.act, M, o.N, o.K, o.qy,
                                      o.sy, o.ws, o.ws_bytes, s)
                 : zq_gemm_w4a8_quant(o.gqx, o.gsx, (const uint8_t *)o.qw,
                                      o.sw, o.G, o.bias, o.act, M, o.N, o.K,
                                      o.qy, o.sy, o.ws, o.ws_bytes, s);
    case kGemmA16:
      return zq_gemm_w8a16(o.x, (const int8_t *)o.qw, o.sw, o.G, o.bias, o.act,
                           M, o.N, o.K, o.y, s);
    case kGemmWs:
      return o.bits == 8
                 ? zq_gemm_w8a8_ws(o.gqx, o.gsx, (const int8_t *)o.qw, o.sw,
                                   o.G, o.bias, o.act, M, o.N, o.K, o.y, o.ws,
                                   o.ws_bytes, s)
                 : zq_gemm_w4a8_ws(o.gqx, o.gsx, (const uint8_t *)o.qw, o.sw,
                                   o.G, o.bias, o.act, M, o.N, o.K, o.y, o.ws,
                                   o.ws_bytes, s);
    case kGemmXq:
      return o.bits == 8
                 ? zq_gemm_w8a8_xq(o.x, (const int8_t *)o.qw, o.sw, o.G,
                                   o.bias, o.act, M, o.N, o.K, o.y, o.qx,
                                   o.sx, s)
                 : zq_gemm_w4a8_xq(o.x, (const uint8_t *)o.qw, o.sw, o.G,
                                   o.bias, o.act, M, o.N, o.K, o.y, o.qx,
                                   o.sx, s);
    case kGemmChunked:
      return o.bits == 8
                 ? zq_gemm_w8a8_chunked(o.gqx, o.gsx, (const int8_t *)o.qw,
                                        o.sw, o.G, o.bias, o.act, M, o.N, o.K,
                                        o.y, s)
                 : zq_gemm_w4a8_chunked(o.gqx, o.gsx, (const uint8_t *)o.qw,
                                        o.sw, o.G, o.bias, o.act, M, o.N, o.K,
                                        o.y, s);
  }
  return zq::fail(ZQ_EINVAL, "zq_chain: unknown call kind");
}

zq_status hip_err(hipError_t e, const char *what) {
  if (e != hipSuccess)
    return zq::fail(ZQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ZQ_OK;
}

}  // namespace

struct zq_chain {
  int max_m = 0;
  std::vector<ChainOp> ops;
  hipStream_t cap = nullptr;  // capture stream (nothing ever runs on it)
  int dev = -1;
  std::vector<GraphEntry> graphs;
  uint64_t tick = 0;
};

namespace {

// Frees a graph once no launch of it can still be in flight.  Its launches
// went to callers' streams, which may be gone by now, so the whole device
// is waited for (this happens only on eviction, a table change or
// destruction; a run records nothing extra on the stream).
void drop(GraphEntry &g) {
  if (g.launched) (void)hipDeviceSynchronize();
  (void)hipGraphExecDestroy(g.exec);
}

// Appends op after checking it as its call would check it over max_m rows
// (the call itself, with M = 0, runs every check but launches nothing).
zq_status add(zq_chain *c, const ChainOp &op, const char *fn,
              bool m_buffers_null) {
  if (!c) return zq::fail(ZQ_EINVAL, "%s: null chain", fn);
  if (m_buffers_null)
    return zq::fail(ZQ_EINVAL, "%s: null buffer sized by M", fn);
  zq_status st = run_op(op, 0, nullptr);
  if (st != ZQ_OK) return st;
  if (op.kind == kGemmChunked && c->max_m > 16)
    return zq::fail(ZQ_EUNSUPPORTED,
                    "%s: the chunked layout serves at most 16 tokens (max_m=%d)",
                    fn, c->max_m);
  if (op.kind == kGemmQuant &&
      op.ws_bytes < zq_gemm_quant_workspace_bytes(c->max_m, op.N))
    return zq::fail(ZQ_EINVAL, "%s: workspace of %zu bytes, %zu needed for %d rows",
                    fn, op.ws_bytes,
                    zq_gemm_quant_workspace_bytes(c->max_m, op.N), c->max_m);
  if (op.kind == kGemmWs) {
    // the largest workspace any token count up to max_m uses
    size_t need = 0;
    for (int m = 1; m <= c->max_m && m <= 64; ++m) {
      const size_t b = zq_gemm_workspace_bytes(m, op.N, op.K, op.bits);
      need = b > need ? b : need;
    }
    if (need > 0 && (!op.ws || op.ws_bytes < need))
      return zq::fail(ZQ_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn,
                      op.ws ? op.ws_bytes : 0, need);
  }
  c->ops.push_back(op);
  return zq::ok();
}

zq_status run_eager(zq_chain *c, int M, void *stream) {
  for (const ChainOp &o : c->ops) {
    const zq_status st = run_op(o, M, stream);
    if (st != ZQ_OK) return st;
  }
  return zq::ok();
}

zq_status check_run(const zq_chain *c, int M, const char *fn) {
  if (!c) return zq::fail(ZQ_EINVAL, "%s: null chain", fn);
  if (M < 0 || M > c->max_m)
    return zq::fail(ZQ_EINVAL, "%s: M=%d outside [0, %d]", fn, M, c->max_m);
  return ZQ_OK;
}

// Captures the chain over M rows into a new graph entry.
zq_status capture(zq_chain *c, int M, GraphEntry *out) {
  const char *fn = "zq_chain_run";
  int dev = 0;
  zq_status st = hip_err(hipGetDevice(&dev), fn);
  if (st != ZQ_OK) return st;
  if (!c->cap) {
    st = hip_err(hipStreamCreateWithFlags(&c->cap, hipStreamNonBlocking), fn);
    if (st != ZQ_OK) return st;
    c->dev = dev;
  } else if (dev != c->dev) {
    return zq::fail(ZQ_EINVAL, "%s: chain captured on device %d, current %d",
                    fn, c->dev, dev);
  }
  st = hip_err(hipStreamBeginCapture(c->cap, hipStreamCaptureModeThreadLocal),
               fn);
  if (st != ZQ_OK) return st;
  const unsigned gen = zq::sched_generation();
  for (const ChainOp &o : c->ops) {
    st = run_op(o, M, c->cap);
    if (st != ZQ_OK) break;
  }
  hipGraph_t graph = nullptr;
  const hipError_t ee = hipStreamEndCapture(c->cap, &graph);
  if (st != ZQ_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  st = hip_err(ee, fn);
  if (st != ZQ_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  hipGraphExec_t exec = nullptr;
  st = hip_err(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0), fn);
  (void)hipGraphDestroy(graph);
  if (st != ZQ_OK) return st;
  *out = GraphEntry{M, gen, exec, false, 0};
  return ZQ_OK;
}

}  // namespace

extern "C" {

zq_status zq_chain_create(int max_m, zq_chain **out) {
  if (!out) return zq::fail(ZQ_EINVAL, "zq_chain_create: null out");
  if (max_m < 1)
    return zq::fail(ZQ_EINVAL, "zq_chain_create: max_m=%d < 1", max_m);
  zq_chain *c = new zq_chain;
  c->max_m = max_m;
  *out = c;
  return zq::ok();
}

zq_status zq_chain_add_ln_quant(zq_chain *c, const void *x_fp16,
                                const void *gamma_fp16, const void *beta_fp16,
                                float eps, int K, int8_t *qx, float *sx,
                                void *ln_out_fp16) {
  ChainOp o{kLnQuant};
  o.x = x_fp16;
  o.gamma = gamma_fp16;
  o.beta = beta_fp16;
  o.eps = eps;
  o.K = K;
  o.qx = qx;
  o.sx = sx;
  o.ln_out = ln_out_fp16;
  return add(c, o, "zq_chain_add_ln_quant", !x_fp16 || !qx || !sx);
}

zq_status zq_chain_add_quant(zq_chain *c, const void *x_fp16, int K,
                             int8_t *qx, float *sx) {
  ChainOp o{kQuant};
  o.x = x_fp16;
  o.K = K;
  o.qx = qx;
  o.sx = sx;
  return add(c, o, "zq_chain_add_quant", !x_fp16 || !qx || !sx);
}

zq_status zq_chain_add_gemm(zq_chain *c, int bits, const int8_t *qx,
                            const float *sx, const void *qw, const float *sw,
                            int G, const void *bias_fp16, int act, int N, int K,
                            void *y_fp16) {
  if (bits != 8 && bits != 4)
    return zq::fail(ZQ_EINVAL, "zq_chain_add_gemm: bits=%d", bits);
  ChainOp o{kGemm};
  o.bits = bits;
  o.gqx = qx;
  o.gsx = sx;
  o.qw = qw;
  o.sw = sw;
  o.G = G;
  o.bias = bias_fp16;
  o.act = act;
  o.N = N;
  o.K = K;
  o.y = y_fp16;
  return add(c, o, "zq_chain_add_gemm", !qx || !sx || !y_fp16);
}

zq_status zq_chain_add_gemm_quant(zq_chain *c, int bits, const int8_t *qx,
                                  const float *sx, const void *qw,
                                  const float *sw, int G, const void *bias_fp16,
                                  int act, int N, int K, int8_t *qy, float *sy,
                                  void *ws, size_t ws_bytes) {
  if (bits != 8 && bits != 4)
    return zq::fail(ZQ_EINVAL, "zq_chain_add_gemm_quant: bits=%d", bits);
  ChainOp o{kGemmQuant};
  o.bits = bits;
  o.gqx = qx;
  o.gsx = sx;
  o.qw = qw;
  o.sw = sw;
  o.G = G;
  o.bias = bias_fp16;
  o.act = act;
  o.N = N;
  o.K = K;
  o.qy = qy;
  o.sy = sy;
  o.ws = ws;
  o.ws_bytes = ws_bytes;
  return add(c, o, "zq_chain_add_gemm_quant", !qx || !sx || !qy || !sy || !ws);
}

zq_status zq_chain_add_gemm_chunked(zq_chain *c, int bits, const int8_t *qx,
                                    const float *sx, const void *qd,
                                    const float *sw, int G,
                                    const void *bias_fp16, int act, int N,
                                    int K, void *y_fp16) {
  if (bits != 8 && bits != 4)
    return zq::fail(ZQ_EINVAL, "zq_chain_add_gemm_chunked: bits=%d", bits);
  ChainOp o{kGemmChunked};
  o.bits = bits;
  o.gqx = qx;
  o.gsx = sx;
  o.qw = qd;
  o.sw = sw;
  o.G = G;
  o.bias = bias_fp16;
  o.act = act;
  o.N = N;
  o.K = K;
  o.y = y_fp16;
  return add(c, o, "zq_chain_add_gemm_chunked", !qx || !sx || !y_fp16);
}

zq_status zq_chain_add_gemm_ws(zq_chain *c, int bits, const int8_t *qx,
                               const float *sx, const void *qw, const float *sw,
                               int G, const void *bias_fp16, int act, int N,
                               int K, void *y_fp16, void *ws, size_t ws_bytes) {
  if (bits != 8 && bits != 4)
    return zq::fail(ZQ_EINVAL, "zq_chain_add_gemm_ws: bits=%d", bits);
  ChainOp o{kGemmWs};
  o.bits = bits;
  o.gqx = qx;
  o.gsx = sx;
  o.qw = qw;
  o.sw = sw;
  o.G = G;
  o.bias = bias_fp16;
  o.act = act;
  o.N = N;
  o.K = K;
  o.y = y_fp16;
  o.ws = ws;
  o.ws_bytes = ws_bytes;
  return add(c, o, "zq_chain_add_gemm_ws", !qx || !sx || !y_fp16);
}

zq_status zq_chain_add_gemm_w8a16(zq_chain *c, const void *x_fp16,
                                  const int8_t *qw, const float *sw, int G,
                                  const void *bias_fp16, int act, int N, int K,
                                  void *y_fp16) {
  ChainOp o{kGemmA16};
  o.x = x_fp16;
  o.qw = qw;
  o.sw = sw;
  o.G = G;
  o.bias = bias_fp16;
  o.act = act;
  o.N = N;
  o.K = K;
  o.y = y_fp16;
  return add(c, o, "zq_chain_add_gemm_w8a16", !x_fp16 || !y_fp16);
}

zq_status zq_chain_add_gemm_xq(zq_chain *c, int bits, const void *x_fp16,
                               const void *qw, const float *sw, int G,
                               const void *bias_fp16, int act, int N, int K,
                               void *y_fp16, int8_t *qx, float *sx) {
  if (bits != 8 && bits != 4)
    return zq::fail(ZQ_EINVAL, "zq_chain_add_gemm_xq: bits=%d", bits);
  ChainOp o{kGemmXq};
  o.bits = bits;
  o.x = x_fp16;
  o.qw = qw;
  o.sw = sw;
  o.G = G;
  o.bias = bias_fp16;
  o.act = act;
  o.N = N;
  o.K = K;
  o.y = y_fp16;
  o.qx = qx;
  o.sx = sx;
  return add(c, o, "zq_chain_add_gemm_xq", !x_fp16 || !y_fp16 || !qx || !sx);
}

zq_status zq_chain_run_eager(zq_chain *c, int M, void *stream) {
  const zq_status st = check_run(c, M, "zq_chain_run_eager");
  if (st != ZQ_OK) return st;
  if (M == 0) return zq::ok();
  return run_eager(c, M, stream);
}

zq_status zq_chain_run(zq_chain *c, int M, void *stream) {
  const char *fn = "zq_chain_run";
  zq_status st = check_run(c, M, fn);
  if (st != ZQ_OK) return st;
  if (M == 0 || c->ops.empty()) return zq::ok();
  // inside a caller's capture: launch directly so the calls join it
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  st = hip_err(hipStreamIsCapturing((hipStream_t)stream, &cs), fn);
  if (st != ZQ_OK) return st;
  if (cs != hipStreamCaptureStatusNone) return run_eager(c, M, stream);

  const unsigned gen = zq::sched_generation();
  GraphEntry *g = nullptr;
  for (size_t i = 0; i < c->graphs.size(); ++i) {
    if (c->graphs[i].M != M) continue;
    if (c->graphs[i].gen == gen) {
      g = &c->graphs[i];
    } else {  // its plans predate the last schedule-table change
      drop(c->graphs[i]);
      c->graphs.erase(c->graphs.begin() + i);
    }
    break;
  }
  if (!g) {
    GraphEntry fresh;
    st = capture(c, M, &fresh);
    if (st != ZQ_OK) return st;
    if ((int)c->graphs.size() >= ZQ_CHAIN_MAX_GRAPHS) {
      size_t lru = 0;
      for (size_t i = 1; i < c->graphs.size(); ++i)
        if (c->graphs[i].last_use < c->graphs[lru].last_use) lru = i;
      drop(c->graphs[lru]);
      c->graphs.erase(c->graphs.begin() + lru);
    }
    c->graphs.push_back(fresh);
    g = &c->graphs.back();
  }
  g->last_use = ++c->tick;
  g->launched = true;
  st = hip_err(hipGraphLaunch(g->exec, (hipStream_t)stream), fn);
  return st == ZQ_OK ? zq::ok() : st;
}

int zq_chain_graphs(const zq_chain *c) { return c ? (int)c->graphs.size() : 0; }

int zq_chain_length(const zq_chain *c) { return c ? (int)c->ops.size() : 0; }

void zq_chain_destroy(zq_chain *c) {
  if (!c) return;
  for (GraphEntry &g : c->graphs) drop(g);
  if (c->cap) (void)hipStreamDestroy(c->cap);
  delete c;
}

}  // extern "C"
