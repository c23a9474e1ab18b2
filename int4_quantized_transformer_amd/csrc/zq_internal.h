// zq_internal.h -- device helpers and internal launcher declarations of
// libzq (gfx950 only).  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "zq.h"

namespace zq {

typedef _Float16 half_t;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// --------------------------------------------------------------- quantizer
// Eq. (2) of the group-wise/token-wise quantizer with S = amax / qmax:
// fp32 IEEE division, clamp to +-qmax, round half to even.  The division
// must stay correctly rounded (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt and without fast-math).
__device__ __forceinline__ int quant_code(float v, float s, float qmax) {
  if (s == 0.0f) return 0;
  float x = v / s;
  x = fminf(fmaxf(x, -qmax), qmax);
  return (int)__builtin_rintf(x);
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

// ------------------------------------------------------------ XCD mapping
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Remap the hardware order so that each XCD receives a contiguous
// range of logical tile ids; the map is a bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int X = 8;
  const int q = total / X, r = total % X;
  const int x = pid % X, i = pid / X;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
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
// Human-readable schedule for (M, N, K, bits); returns chars written.
int describe_gemm_plan(int M, int N, int K, int bits, char *buf, int len);

}  // namespace zq
