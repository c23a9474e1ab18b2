// zq_quant.hip -- quantization kernels of libzq for gfx950.
//
//  * row_quant_kernel: one token row per thread team; LayerNorm (optional)
//    and the token-wise INT8 quantizer fused, the row held in registers
//    (ZeroQuant summary page, Sec. 3.4 "Quantization-Optimized Transformer
//    Kernels": one row per compute unit, scale computed from values already
//    in registers, only INT8 written out; paper App. D, Fig. 2).
//  * weight_quant_kernel: group-wise W8/W4 quantization (Sec. 3.4
//    "Group-wise Weight Quantization", paper Sec. 4.1, Eq. (2)); one
//    workgroup per group of G weight rows, an offline step.
#include "zq_internal.h"

namespace zq {

// ===================================================================== rows
// A team of TPR threads owns one row; each thread holds NCH chunks of 8
// consecutive fp16 values (chunk c = lane + j*TPR covers k = 8c .. 8c+7),
// so global reads are 16-byte per lane and fully coalesced across the team,
// and the int8 writes are 8-byte per lane.  VEC = false is the same
// algorithm with scalar, bounds-checked accesses for K % 8 != 0.
// Teams of 16 or 32 lanes (short rows) put several rows in one wave: the
// rows share the reduction instructions and no lane idles; teams of 256 or
// 1024 threads (long rows, or few rows) reduce through LDS.
template <int TPR>
struct RowTeam {
  static constexpr int kBlock = TPR < 256 ? 256 : TPR;
  static constexpr int kRows = kBlock / TPR;
  static constexpr int kWaves = TPR / kWave;
};

template <int TPR>
__device__ __forceinline__ float team_sum(float v, float *lds) {
  if constexpr (TPR == 16) return rows_of_16_sum(v);
  if constexpr (TPR == 32) {
    v = rows_of_16_sum(v);
    return v + __shfl_xor(v, 16);
  }
  v = wave_sum(v);
  if constexpr (TPR > kWave) {
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
    __syncthreads();
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < TPR / kWave; ++i) s += lds[i];
    v = s;
  }
  return v;
}

template <int TPR>
__device__ __forceinline__ float team_max(float v, float *lds) {
  if constexpr (TPR == 16) return rows_of_16_max(v);
  if constexpr (TPR == 32) {
    v = rows_of_16_max(v);
    return fmaxf(v, __shfl_xor(v, 16));
  }
  v = wave_max(v);
  if constexpr (TPR > kWave) {
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
    __syncthreads();
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < TPR / kWave; ++i) m = fmaxf(m, lds[i]);
    v = m;
  }
  return v;
}

// LayerNorm (optional) and the token-wise quantizer of one row held in
// registers (v, with ok[j] telling which chunks lie inside the row), then
// the stores: codes, the scale and, when asked, the fp16 LayerNorm output.
// hg / hb: this lane's gamma / beta chunks (VEC).  FULL: every chunk of
// every lane lies inside the row (K = 8 NCH TPR), so no chunk is masked.
template <int TPR, int NCH, bool LN, bool VEC, bool FULL = false>
__device__ __forceinline__ void row_finish(
    float (&v)[NCH][8], const bool (&ok)[NCH],
    const half8 (&hg)[LN && VEC ? NCH : 1], const half8 (&hb)[LN && VEC ? NCH : 1],
    const half_t *__restrict__ gamma, const half_t *__restrict__ beta,
    float eps, int K, int tl, int row, float *red, int8_t *__restrict__ qx,
    float *__restrict__ sx, half_t *__restrict__ ln_out) {
  static_assert(VEC || !FULL, "FULL rows take the vector path");
  if constexpr (LN) {
    // mean and biased variance (two passes over the registers, fp32); the
    // centred values v - mean replace v
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[j][i];  // out-of-range values are 0
    const float mean = team_sum<TPR>(s, red) / (float)K;
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      float cs = 0.0f;
      if constexpr (VEC) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[j][i] -= mean;
          cs = fmaf(v[j][i], v[j][i], cs);
        }
        ss += (FULL || ok[j]) ? cs : 0.0f;
      } else {
        // the vector path's arithmetic, element by element (the same bits
        // whenever K % 8 == 0)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = (tl + j * TPR) * 8 + i;
          v[j][i] -= mean;
          cs = (k < K) ? fmaf(v[j][i], v[j][i], cs) : cs;
        }
        ss += cs;
      }
    }
    const float var = team_sum<TPR>(ss, red) / (float)K;
    const float rstd = 1.0f / sqrtf(var + eps);
    // y = (x - mean) rstd gamma + beta, rounded once to the fp16 value the
    // LayerNorm emits (the quantizer takes that value)
    half8 hy[VEC ? NCH : 1];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tl + j * TPR;
      if (!FULL && !ok[j]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = 0.0f;
        continue;
      }
      if constexpr (VEC) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        const u4 gw = __builtin_bit_cast(u4, hg[j]);
        const u4 bw = __builtin_bit_cast(u4, hb[j]);
        u4 yw;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          yw[q] = fma_half2_h(v[j][2 * q] * rstd, v[j][2 * q + 1] * rstd, gw[q],
                              bw[q]);
        hy[j] = __builtin_bit_cast(half8, yw);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = (float)hy[j][i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = c * 8 + i;
          const half_t g = (gamma && k < K) ? gamma[k] : (half_t)1.0f;
          const half_t b = (beta && k < K) ? beta[k] : (half_t)0.0f;
          const float h = (float)fma_half_h(v[j][i] * rstd, g, b);
          v[j][i] = k < K ? h : 0.0f;
        }
      }
    }
    if (ln_out) {
      half_t *lr = ln_out + (size_t)row * K;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = tl + j * TPR;
        if constexpr (VEC) {
          if (FULL || ok[j]) *reinterpret_cast<half8 *>(lr + c * 8) = hy[j];
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (c * 8 + i < K) lr[c * 8 + i] = (half_t)v[j][i];
        }
      }
    }
  }

  // token-wise scale: max |h| / 127 (values past the row end are 0)
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < NCH; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
  const float amax = team_max<TPR>(m, red);
  const Quantizer qz = make_quantizer(amax, 127.0f);
  if (tl == 0) sx[row] = qz.s;

  int8_t *qr = qx + (size_t)row * K;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tl + j * TPR;
    if constexpr (VEC) {
      // amax is the max |v| of this row: the codes need no clamp
      const v2i p = quant8_pack_rowmax(v[j], qz);
      if (FULL || ok[j]) *reinterpret_cast<v2i *>(qr + c * 8) = p;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (c * 8 + i < K) qr[c * 8 + i] = (int8_t)quant_code(v[j][i], qz);
    }
  }
}

// Load one row (chunk j of this lane: k = 8 (tl + j TPR) .. + 7) into v.
template <int TPR, int NCH, bool VEC, bool FULL>
__device__ __forceinline__ void row_load(const half_t *__restrict__ x, int K,
                                         int tl, int row, float (&v)[NCH][8],
                                         bool (&ok)[NCH]) {
  const half_t *xr = x + (size_t)row * K;
  // VEC: chunk j of this lane is either wholly inside the row or wholly
  // past its end (K % 8 == 0); such chunks hold zeros
  // every chunk is loaded (past the row end: the row's last chunk) so that
  // all loads are in flight together, then masked
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tl + j * TPR;
    ok[j] = FULL || c * 8 < K;
    if constexpr (VEC) {
      const int cc = ok[j] ? c : K / 8 - 1;
      const half8 h = *reinterpret_cast<const half8 *>(xr + cc * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = ok[j] ? (float)h[i] : 0.0f;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = c * 8 + i;
        v[j][i] = (k < K) ? (float)xr[k] : 0.0f;
      }
    }
  }
}

// gamma / beta chunks of this lane
template <int TPR, int NCH>
__device__ __forceinline__ void row_affine(const half_t *__restrict__ gamma,
                                           const half_t *__restrict__ beta,
                                           int K, int tl, half8 (&hg)[NCH],
                                           half8 (&hb)[NCH]) {
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tl + j * TPR;
    const int cc = c * 8 < K ? c : K / 8 - 1;
    hg[j] = gamma ? *reinterpret_cast<const half8 *>(gamma + cc * 8)
                  : half8{1, 1, 1, 1, 1, 1, 1, 1};
    hb[j] = beta ? *reinterpret_cast<const half8 *>(beta + cc * 8)
                 : half8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

template <int TPR, int NCH, bool LN, bool VEC, bool FULL>
__global__ void __launch_bounds__(RowTeam<TPR>::kBlock)
row_quant_kernel(const half_t *__restrict__ x, const half_t *__restrict__ gamma,
                 const half_t *__restrict__ beta, float eps, int M, int K,
                 int8_t *__restrict__ qx, float *__restrict__ sx,
                 half_t *__restrict__ ln_out) {
  using T = RowTeam<TPR>;
  __shared__ float red[TPR > kWave ? TPR / kWave : 1];
  const int team = threadIdx.x / TPR;
  const int tl = threadIdx.x % TPR;
  const int row = blockIdx.x * T::kRows + team;
  // A row past the end retires its whole team (16 or 32 lanes of a wave, a
  // wave, or with TPR > 64 the entire block), so every cross-lane step of
  // a live team reads live lanes only.
  if (row >= M) return;

  float v[NCH][8];
  bool ok[NCH];
  row_load<TPR, NCH, VEC, FULL>(x, K, tl, row, v, ok);
  // LayerNorm weight and bias chunks: requested with the row, so that their
  // latency overlaps the row's instead of following the two reductions
  half8 hg[LN && VEC ? NCH : 1], hb[LN && VEC ? NCH : 1];
  if constexpr (LN && VEC) row_affine<TPR, NCH>(gamma, beta, K, tl, hg, hb);
  row_finish<TPR, NCH, LN, VEC, FULL>(v, ok, hg, hb, gamma, beta, eps, K, tl,
                                      row, red, qx, sx, ln_out);
}

template <int TPR, int NCH, bool LN, bool VEC>
static hipError_t launch_rows(const half_t *x, const half_t *g,
                              const half_t *b, float eps, int M, int K,
                              int8_t *qx, float *sx, half_t *ln_out,
                              hipStream_t s) {
  using T = RowTeam<TPR>;
  const int grid = (M + T::kRows - 1) / T::kRows;
  // rows that fill every lane's chunks exactly (768 with 16 lanes, 4096 or
  // 6144 with 256 threads, ...) skip the chunk masks
  if (VEC && K == 8 * NCH * TPR)
    hipLaunchKernelGGL((row_quant_kernel<TPR, NCH, LN, VEC, VEC>), dim3(grid),
                       dim3(T::kBlock), 0, s, x, g, b, eps, M, K, qx, sx,
                       ln_out);
  else
    hipLaunchKernelGGL((row_quant_kernel<TPR, NCH, LN, VEC, false>), dim3(grid),
                       dim3(T::kBlock), 0, s, x, g, b, eps, M, K, qx, sx,
                       ln_out);
  return hipGetLastError();
}

template <int TPR, bool LN, bool VEC>
static hipError_t dispatch_nch(int nch, const half_t *x, const half_t *g,
                               const half_t *b, float eps, int M, int K,
                               int8_t *qx, float *sx, half_t *ln_out,
                               hipStream_t s) {
  if constexpr (TPR == 64) {  // one wave per row of up to 6144 elements
    if (nch > 8)
      return launch_rows<TPR, 12, LN, VEC>(x, g, b, eps, M, K, qx, sx, ln_out, s);
  }
  switch (nch) {
    case 1: return launch_rows<TPR, 1, LN, VEC>(x, g, b, eps, M, K, qx, sx, ln_out, s);
    case 2: return launch_rows<TPR, 2, LN, VEC>(x, g, b, eps, M, K, qx, sx, ln_out, s);
    case 3: return launch_rows<TPR, 3, LN, VEC>(x, g, b, eps, M, K, qx, sx, ln_out, s);
    case 4: return launch_rows<TPR, 4, LN, VEC>(x, g, b, eps, M, K, qx, sx, ln_out, s);
    case 6: return launch_rows<TPR, 6, LN, VEC>(x, g, b, eps, M, K, qx, sx, ln_out, s);
    default: return launch_rows<TPR, 8, LN, VEC>(x, g, b, eps, M, K, qx, sx, ln_out, s);
  }
}

template <bool LN, bool VEC>
static hipError_t dispatch_tpr(const half_t *x, const half_t *g,
                               const half_t *b, float eps, int M, int K,
                               int8_t *qx, float *sx, half_t *ln_out,
                               hipStream_t s) {
  // Rows of 1024 or more elements: the smallest team that holds the row in
  // at most 2 chunks of 8 per thread (a sweep of team sizes at 2048 - 8192
  // tokens found these faster than fewer, fuller threads: 8192 x 1024 LN
  // 11.2 -> 9.8 us, 4096 x 3072 10.7 -> 9.8 us), except that a 256-thread
  // team keeps rows of up to 4 chunks per thread rather than spreading them
  // over 1024 threads (2048 x 6144 LN: 22.4 us with 1024 threads of one
  // chunk, 13.3 us with 256 threads of three; one token of 6144: 4.0 ->
  // 3.2 us).  Shorter rows: the smallest team that holds the row in at most
  // 8 chunks (16 lanes for 768 elements: several rows per wave share the
  // reduction instructions); then, while fewer than 1024 waves would run,
  // larger teams (down to 2 chunks per thread) so that a few rows still
  // spread over the device.  (Teams that own several rows and request them
  // all before finishing the first measured slower at every shape tried.)
  const int chunks = (K + 7) / 8;
  auto next = [](int t) { return t < 64 ? 2 * t : 4 * t; };
  const int cap = chunks >= 128 ? 2 : 8;
  int tpr = 16;
  while (tpr < 1024 && (chunks + tpr - 1) / tpr > cap &&
         !(tpr == 256 && (chunks + 255) / 256 <= 4))
    tpr = next(tpr);
  while (tpr < 1024 && (long)M * tpr < 1024L * 64 && chunks >= 2 * next(tpr))
    tpr = next(tpr);
  // ZQ_ROW_TPR=<16|32|64|256|1024> forces the team size where the row fits
  // (tuning aid)
  static const int forced = [] {
    const char *e = getenv("ZQ_ROW_TPR");
    return e ? atoi(e) : 0;
  }();
  if ((forced == 16 || forced == 32 || forced == 64 || forced == 256 ||
       forced == 1024) &&
      (chunks + forced - 1) / forced <= (forced == 64 ? 12 : 8))
    tpr = forced;
  const int per = (chunks + tpr - 1) / tpr;
  const int nch = per <= 4 ? per : (per <= 6 ? 6 : (per <= 8 ? 8 : 12));
  if (tpr == 16) return dispatch_nch<16, LN, VEC>(nch, x, g, b, eps, M, K, qx, sx, ln_out, s);
  if (tpr == 32) return dispatch_nch<32, LN, VEC>(nch, x, g, b, eps, M, K, qx, sx, ln_out, s);
  if (tpr == 64) return dispatch_nch<64, LN, VEC>(nch, x, g, b, eps, M, K, qx, sx, ln_out, s);
  if (tpr == 256) return dispatch_nch<256, LN, VEC>(nch, x, g, b, eps, M, K, qx, sx, ln_out, s);
  return dispatch_nch<1024, LN, VEC>(nch, x, g, b, eps, M, K, qx, sx, ln_out, s);
}

hipError_t launch_row_quant(const void *x, const void *gamma, const void *beta,
                            float eps, int M, int K, bool ln, int8_t *qx,
                            float *sx, void *ln_out, hipStream_t s) {
  const half_t *xh = static_cast<const half_t *>(x);
  const half_t *g = static_cast<const half_t *>(gamma);
  const half_t *b = static_cast<const half_t *>(beta);
  half_t *lo = static_cast<half_t *>(ln_out);
  // the vector path reads x, gamma and beta as 16-byte chunks and writes
  // 8-byte code chunks
  const bool vec = (K % 8 == 0) && ((uintptr_t)x % 16 == 0) &&
                   ((uintptr_t)qx % 8 == 0) &&
                   (!lo || (uintptr_t)lo % 16 == 0) &&
                   (!g || (uintptr_t)g % 16 == 0) &&
                   (!b || (uintptr_t)b % 16 == 0);
  if (ln)
    return vec ? dispatch_tpr<true, true>(xh, g, b, eps, M, K, qx, sx, lo, s)
               : dispatch_tpr<true, false>(xh, g, b, eps, M, K, qx, sx, lo, s);
  return vec ? dispatch_tpr<false, true>(xh, g, b, eps, M, K, qx, sx, lo, s)
             : dispatch_tpr<false, false>(xh, g, b, eps, M, K, qx, sx, lo, s);
}

// ============================================================ static range
// The prior-PTQ scheme that token-wise scales replace (summary page,
// Sec. 3.4 "Token-wise Activation Quantization"; paper App. B.1): one
// activation range per tensor, calibrated offline as a moving average of
// batch minima and maxima, then frozen.
//  * calibrate_kernel (offline): one workgroup reduces the batch's min and
//    max (exact, independent of order), then updates state = {x_min, x_max}:
//    the first batch initializes, later ones move it by
//    x = m * x + (1 - m) * batch, in fp32 with each product and the sum
//    rounded separately.
//  * static_quant_kernel: Eq. (2) over the whole tensor with
//    S = max(|x_min|, |x_max|) / 127 taken from the device-side state; values
//    beyond the calibrated range clamp to +-127.
constexpr int kCalThreads = 1024;

__global__ void __launch_bounds__(kCalThreads)
calibrate_kernel(const half_t *__restrict__ x, size_t n, float momentum,
                 int first, float *__restrict__ state) {
  __shared__ float rmn[kCalThreads / kWave], rmx[kCalThreads / kWave];
  float mn = INFINITY, mx = -INFINITY;
  if (((uintptr_t)x & 15) == 0) {
    const size_t n8 = n / 8;
    for (size_t c = threadIdx.x; c < n8; c += kCalThreads) {
      const half8 h = *reinterpret_cast<const half8 *>(x + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = (float)h[e];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
      }
    }
    for (size_t k = n8 * 8 + threadIdx.x; k < n; k += kCalThreads) {
      const float v = (float)x[k];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
  } else {
    for (size_t k = threadIdx.x; k < n; k += kCalThreads) {
      const float v = (float)x[k];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
  }
  mn = -wave_max(-mn);
  mx = wave_max(mx);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    rmn[w] = mn;
    rmx[w] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bmn = rmn[0], bmx = rmx[0];
    for (int i = 1; i < kCalThreads / kWave; ++i) {
      bmn = fminf(bmn, rmn[i]);
      bmx = fmaxf(bmx, rmx[i]);
    }
    if (first) {
      state[0] = bmn;
      state[1] = bmx;
    } else {
#pragma clang fp contract(off)
      const float wgt = 1.0f - momentum;
      const float a0 = momentum * state[0], b0 = wgt * bmn;
      const float a1 = momentum * state[1], b1 = wgt * bmx;
      state[0] = a0 + b0;
      state[1] = a1 + b1;
    }
  }
}

__global__ void __launch_bounds__(256)
static_quant_kernel(const half_t *__restrict__ x, size_t n,
                    const float *__restrict__ state, int8_t *__restrict__ q,
                    float *__restrict__ s_out, int vec) {
  const Quantizer z =
      make_quantizer(fmaxf(fabsf(state[0]), fabsf(state[1])), 127.0f);
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nth = (size_t)gridDim.x * blockDim.x;
  if (tid == 0) *s_out = z.s;
  size_t done = 0;
  if (vec) {
    const size_t n8 = n / 8;
    for (size_t c = tid; c < n8; c += nth) {
      const half8 h = *reinterpret_cast<const half8 *>(x + c * 8);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)h[e];
      *reinterpret_cast<v2i *>(q + c * 8) = quant8_pack(v, z);
    }
    done = n8 * 8;
  }
  for (size_t k = done + tid; k < n; k += nth)
    q[k] = (int8_t)quant_code((float)x[k], z);
}

hipError_t launch_calibrate(const void *x, size_t n, float momentum, int first,
                            float *state, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(1), dim3(kCalThreads), 0, s,
                     static_cast<const half_t *>(x), n, momentum, first, state);
  return hipGetLastError();
}

hipError_t launch_static_quant(const void *x, size_t n, const float *state,
                               int8_t *q, float *s_out, hipStream_t s) {
  const int vec = (((uintptr_t)x & 15) == 0) && (((uintptr_t)q & 7) == 0);
  const size_t chunks = (n + 7) / 8;
  size_t blocks = (chunks + 255) / 256;
  if (blocks > 4096) blocks = 4096;  // grid-stride beyond
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(static_quant_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     s, static_cast<const half_t *>(x), n, state, q, s_out, vec);
  return hipGetLastError();
}

// ================================================================= weights
constexpr int kWQThreads = 1024;

template <bool VEC>
__global__ void __launch_bounds__(kWQThreads)
weight_quant_kernel(const half_t *__restrict__ w, int K, int G, int bits,
                    void *__restrict__ qw, float *__restrict__ sw) {
  __shared__ float red[kWQThreads / kWave];
  const int g = blockIdx.x;
  const size_t n = (size_t)G * K;        // elements in the group
  const half_t *src = w + (size_t)g * n;
  const float qmax = bits == 8 ? 127.0f : 7.0f;

  // pass 1: group amax
  float m = 0.0f;
  if constexpr (VEC) {
    for (size_t i = (size_t)threadIdx.x * 8; i < n; i += (size_t)kWQThreads * 8) {
      half8 h = *reinterpret_cast<const half8 *>(src + i);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)h[e]));
    }
  } else {
    for (size_t i = threadIdx.x; i < n; i += kWQThreads)
      m = fmaxf(m, fabsf((float)src[i]));
  }
  m = wave_max(m);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kWQThreads / kWave; ++i) amax = fmaxf(amax, red[i]);
  const Quantizer qz = make_quantizer(amax, qmax);
  if (threadIdx.x == 0) sw[g] = qz.s;

  // pass 2: codes
  if (bits == 8) {
    int8_t *dst = static_cast<int8_t *>(qw) + (size_t)g * n;
    if constexpr (VEC) {
      for (size_t i = (size_t)threadIdx.x * 8; i < n; i += (size_t)kWQThreads * 8) {
        half8 h = *reinterpret_cast<const half8 *>(src + i);
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = quant_code((float)h[e], qz);
        v2i p;
        p[0] = (int)pack4_i8(q[0], q[1], q[2], q[3]);
        p[1] = (int)pack4_i8(q[4], q[5], q[6], q[7]);
        *reinterpret_cast<v2i *>(dst + i) = p;
      }
    } else {
      for (size_t i = threadIdx.x; i < n; i += kWQThreads)
        dst[i] = (int8_t)quant_code((float)src[i], qz);
    }
  } else {
    // K is even, so element pairs (2j, 2j+1) of the flattened group are
    // the (even k, odd k) pairs of one row: low nibble = even k.
    uint8_t *dst = static_cast<uint8_t *>(qw) + (size_t)g * (n / 2);
    if constexpr (VEC) {
      for (size_t i = (size_t)threadIdx.x * 8; i < n; i += (size_t)kWQThreads * 8) {
        half8 h = *reinterpret_cast<const half8 *>(src + i);
        uint32_t p = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          p |= (uint32_t)(quant_code((float)h[e], qz) & 0xF) << (4 * e);
        *reinterpret_cast<uint32_t *>(dst + i / 2) = p;
      }
    } else {
      for (size_t j = threadIdx.x; j < n / 2; j += kWQThreads) {
        const int lo = quant_code((float)src[2 * j], qz) & 0xF;
        const int hi = quant_code((float)src[2 * j + 1], qz) & 0xF;
        dst[j] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

hipError_t launch_quantize_weights(const void *w, int N, int K, int G,
                                   int bits, void *qw, float *sw,
                                   hipStream_t s) {
  const size_t n = (size_t)G * K;
  const bool vec = (n % 8 == 0) && ((uintptr_t)w % 16 == 0) &&
                   ((uintptr_t)qw % 8 == 0);
  const half_t *wh = static_cast<const half_t *>(w);
  if (vec)
    hipLaunchKernelGGL(weight_quant_kernel<true>, dim3(N / G), dim3(kWQThreads),
                       0, s, wh, K, G, bits, qw, sw);
  else
    hipLaunchKernelGGL(weight_quant_kernel<false>, dim3(N / G),
                       dim3(kWQThreads), 0, s, wh, K, G, bits, qw, sw);
  return hipGetLastError();
}

}  // namespace zq
