// zq_internal.h -- device helpers and internal launcher declarations of
// libzq (gfx950 only).  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "zq.h"

#define ZQ_HD __host__ __device__
#include "zq_index.h"

namespace zq {

typedef _Float16 half_t;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- reductions
// Wave-wide all-reduce with DPP lane permutes inside each row of 16 lanes
// (quad_perm, half-row mirror, row mirror) and v_readlane for the four
// rows, instead of LDS-routed shuffles.  The sum's association order is
// fixed, so results are deterministic.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, false));
}

__device__ __forceinline__ float rows_of_16_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ float rows_of_16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}

__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = rows_of_16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = rows_of_16_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)),
               fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// --------------------------------------------------------------- quantizer
// Eq. (2) of the group-wise/token-wise quantizer with S = amax / qmax:
// q = rint(clamp(v / S, -qmax, qmax)) with the fp32 IEEE quotient v / S
// and round half to even.
//
// Fast evaluation with identical results: with r = fl(1 / S) (IEEE) and
// q0 = fl(v * r), |q0 - v/S| <= |v/S| * 2^-23 (two roundings of relative
// size 2^-24), and fl(v/S) is within |v/S| * 2^-24 of v/S, so
// |q0 - fl(v/S)| <= 3 * 2^-24 * |v/S| < 2.3e-5 for |v/S| <= 128.  The
// integer rint(clamp(.)) can only differ between q0 and fl(v/S) if a
// half-integer lies between them, i.e. if q0 is within 2.3e-5 of k + 0.5;
// in that case (rare: about 6e-5 of the values) the exact division is
// evaluated.  The library is built with -fhip-fp32-correctly-rounded-
// divide-sqrt and without fast-math, so both divisions are IEEE.
struct Quantizer {
  float s;    // scale S
  float r;    // fl(1 / S)
  float qmax;
};

__device__ __forceinline__ Quantizer make_quantizer(float amax, float qmax) {
  Quantizer z;
  z.qmax = qmax;
  z.s = amax / qmax;
  z.r = z.s == 0.0f ? 0.0f : 1.0f / z.s;
  return z;
}

__device__ __forceinline__ int quant_code(float v, const Quantizer &z) {
  if (z.s == 0.0f) return 0;
  float x = v * z.r;
  const float d = x - floorf(x);
  if (fabsf(d - 0.5f) <= 3.0517578125e-05f) x = v / z.s;  // 2^-15 margin
  x = fminf(fmaxf(x, -z.qmax), z.qmax);
  return (int)__builtin_rintf(x);
}

// Eight values at once, with the same results as quant_code: q0 = rint(x)
// for x = fl(v * r), and the eight are redone with the IEEE division when
// d = fma(v, r, -q0) (v*r - q0 rounded once) has |d| >= 0.5 - 2^-15.  d
// differs from x - q0 by at most half an ulp of x plus half an ulp of d,
// under 3.9e-6 for |x| <= 128, so every x within 2.3e-5 of a half-integer
// (the only x whose code can differ from that of fl(v/S), see above) has
// |d| > 0.5 - 2.7e-5 and is redone.  rint is monotonic and +-qmax are
// integers, so clamping after rounding gives the same integers as clamping
// before.  The codes are returned as two's-complement bytes, value i in
// byte i.
__device__ __forceinline__ v2i quant8_pack(const float (&v)[8],
                                           const Quantizer &z) {
  float q[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    q[i] = __builtin_rintf(v[i] * z.r);  // S == 0: r == 0, every code 0
    const float d = __builtin_fmaf(v[i], z.r, -q[i]);
    near |= fabsf(d) >= 0.499969482421875f;  // 0.5 - 2^-15
  }
  if (near) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_rintf(v[i] / z.s);
  }
  int c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    c[i] = (int)__builtin_amdgcn_fmed3f(q[i], -z.qmax, z.qmax);
  // bytes: perm selector 0x0c yields zero, 0-3 bytes of the second
  // operand, 4-7 bytes of the first
  v2i r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = __builtin_amdgcn_perm((uint32_t)c[4 * h + 1],
                                              (uint32_t)c[4 * h], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm((uint32_t)c[4 * h + 3],
                                              (uint32_t)c[4 * h + 2], 0x0c0c0400u);
    r[h] = (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
  }
  return r;
}

// quant8_pack for values whose scale comes from their own row: amax is the
// max |v| over a set of values that includes these eight.  Same codes as
// quant8_pack, with fewer instructions:
//  * no clamp: |v| <= amax gives |v * r| <= 127 (1 + 2^-24)^2 < 127.5 (S
//    and r each round with relative error <= 2^-24), and likewise
//    |fl(v / S)| < 127.5, so every code is in [-127, 127] already;
//  * one rounding step: t = fma(v, r, 1.5 * 2^23) is 1.5 * 2^23 + RNE(v r)
//    of the exact product v r (|v r| < 2^22, so t's unit is 1), its low
//    byte is that integer in two's complement, and f = t - 1.5 * 2^23 is
//    the integer exactly.  RNE(v r) and quant8_pack's rint(fl(v r)) can
//    differ only if v r lies within |v r| 2^-24 <= 7.6e-6 of a
//    half-integer; then d = fma(v, r, -f) (v r - f, rounded once) has
//    |d| > 0.5 - 2^-15 and the eight values are redone with the IEEE
//    division, the same test and fallback as quant8_pack's (whose own
//    margin, 2.3e-5, the same threshold covers).
__device__ __forceinline__ v2i quant8_pack_rowmax(const float (&v)[8],
                                                  const Quantizer &z) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  float t[8];
  float dm = 0.0f;  // max |d| of the eight (one compare instead of eight)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    t[i] = __builtin_fmaf(v[i], z.r, kMagic);  // S == 0: r == 0, code 0
    const float d = __builtin_fmaf(v[i], z.r, -(t[i] - kMagic));
    dm = fmaxf(dm, fabsf(d));
  }
  if (dm >= 0.499969482421875f) {  // 0.5 - 2^-15
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = __builtin_rintf(v[i] / z.s) + kMagic;
  }
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = __builtin_bit_cast(uint32_t, t[i]);
  v2i r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = __builtin_amdgcn_perm(c[4 * h + 1], c[4 * h], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(c[4 * h + 3], c[4 * h + 2], 0x0c0c0400u);
    r[h] = (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
  }
  return r;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) |
         ((uint32_t)(c & 0xff) << 16) | ((uint32_t)(d & 0xff) << 24);
}

// ------------------------------------------------------------------- GeLU
// GeLU(z) = z * Phi(z), the exact (erf) form, evaluated as
//   z * sigmoid(z * P(min(z^2, 36)))
// where P is a degree-4 polynomial fitted (iteratively reweighted least
// squares on |z| <= 6) so that z * P(z^2) = logit(Phi(z)).  In fp32 the
// result is within 3.5e-6 of z * Phi(z) for all z (checked on |z| <= 60;
// beyond |z| = 6 the sigmoid is saturated: Phi differs from 0 or 1 by less
// than 1e-9).  Coefficients below are -log2(e) * P so that
// sigmoid(x) = 1 / (1 + 2^(-x log2 e)) needs one exp2 and one rcp.
__device__ __forceinline__ float gelu_erf(float z) {
  const float u = fminf(z * z, 36.0f);
  float q = fmaf(u, -3.2104740057548042e-06f, 8.791135769570246e-05f);
  q = fmaf(u, q, 0.0003620403294917196f);
  q = fmaf(u, q, -0.10522996634244919f);
  q = fmaf(u, q, -2.3020436763763428f);
  const float e = __builtin_amdgcn_exp2f(z * q);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// ------------------------------------------------------- fp16 epilogue out
// Every GEMM epilogue produces its fp16 output through these two helpers, so
// that the output bits do not depend on the kernel, the tile or on what the
// compiler contracts (HIP contracts a*b+c and may fold a product and the
// fp16 conversion into one mixed-precision fma, which rounds once instead
// of twice):
//  * no activation: y = a * s + b rounded once, to nearest even, from the
//    exact value (v_fma_mix{lo,hi}_f16 with a, s as fp32 and b as fp16);
//  * GeLU: the fp32 value z = fma(a, s, b), GeLU in fp32, then rounded to
//    fp16 (the GeLU result is made opaque first, so its last product is
//    never folded into the conversion).
// Two outputs a_i * s + b_i packed low / high; bb holds b_0 low, b_1 high.
__device__ __forceinline__ uint32_t fma_half2(float a0, float a1, float s,
                                              uint32_t bb) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %3, %4 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %2, %3, %4 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(r)
      : "v"(a0), "v"(a1), "v"(s), "v"(bb));
  return r;
}

// LayerNorm's affine step for two values: fp16(a_i * g_i + b_i) rounded
// once from the exact value, with g and b read as fp16 pairs (low: value 0,
// high: value 1) straight from their registers.
__device__ __forceinline__ uint32_t fma_half2_h(float a0, float a1, uint32_t gg,
                                                uint32_t bb) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %3, %4 op_sel_hi:[0,1,1]\n\t"
      "v_fma_mixhi_f16 %0, %2, %3, %4 op_sel:[0,1,1] op_sel_hi:[0,1,1]"
      : "=&v"(r)
      : "v"(a0), "v"(a1), "v"(gg), "v"(bb));
  return r;
}

// The same for one value: fp16(a * g + b), g and b fp16, rounded once.
__device__ __forceinline__ half_t fma_half_h(float a, half_t g, half_t b) {
  const uint32_t gg = __builtin_bit_cast(uint16_t, g);
  const uint32_t bb = __builtin_bit_cast(uint16_t, b);
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,1,1]"
      : "=v"(r)
      : "v"(a), "v"(gg), "v"(bb));
  return __builtin_bit_cast(half_t, (uint16_t)r);
}

__device__ __forceinline__ half_t fma_half(float a, float s, half_t b) {
  const uint32_t bb = __builtin_bit_cast(uint16_t, b);
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,0,1]"
      : "=v"(r)
      : "v"(a), "v"(s), "v"(bb));
  return __builtin_bit_cast(half_t, (uint16_t)r);
}

__device__ __forceinline__ half_t gelu_half(float a, float s, half_t b) {
  float g = gelu_erf(fmaf(a, s, (float)b));
  asm("" : "+v"(g));
  return (half_t)g;
}


// Launchers (defined in the .hip files); they return hipSuccess or the
// error of the launch.  Arguments are already validated.
hipError_t launch_quantize_weights(const void *w, int N, int K, int G,
                                   int bits, void *qw, float *sw,
                                   hipStream_t s);
hipError_t launch_row_quant(const void *x, const void *gamma,
                            const void *beta, float eps, int M, int K,
                            bool ln, int8_t *qx, float *sx, void *ln_out,
                            hipStream_t s);

struct GemmArgs {
  const int8_t *qx;
  const float *sx;
  const void *qw;  // int8 [N][K] or packed uint8 [N][K/2]
  const float *sw;
  const half_t *bias;
  void *out;       // fp16 y or int32 acc
  int G, M, N, K;
  int act;         // 0 none, 1 GeLU
  int bits;        // 8 or 4
  bool raw_i32;    // write int32 acc instead of the fused epilogue
};

hipError_t launch_gemm(const GemmArgs &a, hipStream_t s);
// The linear of an fp16 activation (a.qx holds fp16 [M][K], a.sx unused):
// token-wise codes qx [M][K] and scales sx [M] written for the caller, and
// y = the GEMM of those codes (one kernel for one token where the plan is
// the GEMV, else the row quantizer and the plan's kernel).
hipError_t launch_gemm_xq(const GemmArgs &a, int8_t *qx, float *sx,
                          hipStream_t s);
int describe_gemm_xq_plan(int M, int N, int K, int bits, char *buf, int len);
// The GEMM's fp16 output quantized token-wise (codes qy [M][N], scales sy
// [M]) for the next linear; ws: caller workspace of gemm_quant_ws_bytes.
hipError_t launch_gemm_quant(const GemmArgs &a, int8_t *qy, float *sy,
                             void *ws, hipStream_t s);
size_t gemm_quant_ws_bytes(int M, int N);
// Static per-tensor range: one calibration step (state = {x_min, x_max}) and
// the frozen-scale quantizer (s_out: S).
hipError_t launch_calibrate(const void *x, size_t n, float momentum, int first,
                            float *state, hipStream_t s);
hipError_t launch_static_quant(const void *x, size_t n, const float *state,
                               int8_t *q, float *s_out, hipStream_t s);
// INT8 weights with fp16 activations (a.qx holds fp16 [M][K], a.sx unused).
hipError_t launch_gemm_w8a16(const GemmArgs &a, hipStream_t s);
// Chunk-contiguous weight layout of the rings of up to 16 token rows:
// its row-block and chunk sizes for the shape (false: the shape does not
// tile), the repack, and the GEMM over it (1 <= M <= 16).
bool chunked_layout(int N, int K, int bits, int *bn, int *ck, int *xr);
hipError_t launch_pack_chunked(const void *qw, int N, int K, int bits,
                               void *out, hipStream_t s);
hipError_t launch_gemm_chunked(const GemmArgs &a, hipStream_t s);
int describe_gemm_chunked_plan(int M, int N, int K, int bits, char *buf,
                               int len);
int describe_gemm_w8a16_plan(int M, int N, int K, char *buf, int len);
// Human-readable schedule for (M, N, K, bits); returns chars written.
int describe_gemm_plan(int M, int N, int K, int bits, char *buf, int len);
// With a caller workspace (gemm_ws_bytes of it): decode-sized M over few
// weight tiles splits K over several workgroups per tile plus a reduction
// kernel; otherwise the same launches as launch_gemm.
size_t gemm_ws_bytes(int M, int N, int K, int bits);
hipError_t launch_gemm_ws(const GemmArgs &a, void *ws, hipStream_t s);
int describe_gemm_ws_plan(int M, int N, int K, int bits, char *buf, int len);

// Schedule table (bits, N, K, M range) -> plan, consulted before the
// built-in rules.  tune_gemm times every applicable plan at each M of ms[]
// (ascending, buffers of base sized for the last) and stores the fastest
// for (previous M, M]; chosen_kind/cfg/us (nm entries, may be null) report
// what it picked.  The generation changes with every edit.
hipError_t tune_gemm(const GemmArgs &base, const int *ms, int nm, int reps,
                     hipStream_t s, int *chosen_kind, int *chosen_cfg,
                     float *chosen_us);
unsigned sched_generation();
void sched_clear();
int sched_entries();
size_t sched_export(char *buf, size_t len);  // returns bytes needed (with NUL)
int sched_import(const char *text);          // entries added, or -(bad line)

// Error reporting of the C ABI (the thread-local zq_last_error string).
zq_status fail(zq_status st, const char *fmt, ...);
zq_status ok();

}  // namespace zq
