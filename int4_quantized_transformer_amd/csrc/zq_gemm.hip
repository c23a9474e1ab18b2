// zq_gemm.hip -- INT8 x INT8 GEMM with fused dequantization for gfx950.
//
// ZeroQuant summary page, Sec. 3.4 "Quantization-Optimized Transformer
// Kernels" (paper Sec. 4.3, App. D): an INT8 GEMM whose epilogue turns the
// INT32 accumulator into fp16 with the per-token activation scale and the
// per-group weight scale (read before the main loop ends), so that no
// separate dequantization kernel runs; the tiling is picked per token count
// (throughput-oriented for large batches, bandwidth-oriented for small).
//
// Both kernels use v_mfma_i32_16x16x64_i8.  The weight tile is the MFMA
// "A" operand (rows = output features n) and the activation tile the "B"
// operand (columns = tokens t), so each lane ends with 4 consecutive n of
// one token: y[t][n..n+3] is one 8-byte store.  Within one MFMA the
// assignment of k to (lane group, byte) only has to agree between the two
// operands, since the integer sum does not depend on the order of k.
//
// W4: a packed byte holds (even k, odd k) in its (low, high) nibble.  Masking
// a 32-bit word with 0xF0F0F0F0 (after a 4-bit left shift for the low
// nibbles) gives bytes equal to 16*q, two's complement, with the even k in
// one word and the odd k in the other; the activation bytes are permuted
// into the same (even, odd) order, the MFMA accumulates 16*acc, and the
// result is shifted right by 4 (exact: every product is a multiple of 16).
#include <stdio.h>

#include "zq_internal.h"

namespace zq {

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 8 packed W4 bytes (k = 0..15) -> 16 bytes of 16*q in the order
// [k0 k2 k4 k6 | k1 k3 k5 k7 | k8 k10 k12 k14 | k9 k11 k13 k15].
__device__ __forceinline__ v4i unpack_w4(int d0, int d1) {
  v4i r;
  r[0] = (int)(((uint32_t)d0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)((uint32_t)d0 & 0xF0F0F0F0u);
  r[2] = (int)(((uint32_t)d1 << 4) & 0xF0F0F0F0u);
  r[3] = (int)((uint32_t)d1 & 0xF0F0F0F0u);
  return r;
}

// 16 activation bytes (k = 0..15) -> the same (even, odd) order.
__device__ __forceinline__ v4i perm_even_odd(v4i x) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm((uint32_t)x[1], (uint32_t)x[0], 0x06040200u);
  r[1] = (int)__builtin_amdgcn_perm((uint32_t)x[1], (uint32_t)x[0], 0x07050301u);
  r[2] = (int)__builtin_amdgcn_perm((uint32_t)x[3], (uint32_t)x[2], 0x06040200u);
  r[3] = (int)__builtin_amdgcn_perm((uint32_t)x[3], (uint32_t)x[2], 0x07050301u);
  return r;
}

__device__ __forceinline__ v4i ld16(const void *p) {
  return *reinterpret_cast<const v4i *>(p);
}

// ---------------------------------------------------------------- epilogue
// Lane holds acc for n = nb + r (r = 0..3) at token t.  Fused path:
// y = fp16(act(float(acc) * (sx[t] * sw[n / G]) + bias[n])).
template <bool W4, bool RAW>
__device__ __forceinline__ void store_quad(const GemmArgs &p, int t, int nb,
                                           v4i acc, float sxt) {
  if (t >= p.M || nb >= p.N) return;
  if constexpr (W4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] >>= 4;
  }
  if constexpr (RAW) {
    int32_t *o = static_cast<int32_t *>(p.out) + (size_t)t * p.N + nb;
    if (nb + 3 < p.N && (p.N & 3) == 0) {
      *reinterpret_cast<v4i *>(o) = acc;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nb + r < p.N) o[r] = acc[r];
    }
  } else {
    half4 h;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = nb + r < p.N ? nb + r : p.N - 1;
      float z = (float)acc[r] * (sxt * p.sw[n / p.G]);
      if (p.bias) z += (float)p.bias[n];
      if (p.act == ZQ_ACT_GELU) z = gelu_erf(z);
      h[r] = (half_t)z;
    }
    half_t *o = static_cast<half_t *>(p.out) + (size_t)t * p.N + nb;
    if (nb + 3 < p.N && (p.N & 3) == 0) {
      *reinterpret_cast<half4 *>(o) = h;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nb + r < p.N) o[r] = h[r];
    }
  }
}

// =================================================================== tiled
// Block tile BN (n) x BM (t) x BK (k bytes of activation per stage),
// waves arranged (BN/WN) x (BM/WM), each wave WN x WM with 16x16 MFMA
// fragments.  Global -> registers -> LDS with double buffering: the loads
// for stage k+1 are in flight while stage k is multiplied.  LDS rows are
// padded by 16 bytes so that the 16-byte fragment reads of 8 consecutive
// rows hit disjoint banks.
template <int BN_, int BM_, int WN_, int WM_, bool W4_>
struct Tile {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_;
  static constexpr bool W4 = W4_;
  static constexpr int BK = 128;
  static constexpr int NWN = BN / WN, NWM = BM / WM;
  static constexpr int NWAVES = NWN * NWM, NT = NWAVES * kWave;
  static constexpr int FN = WN / 16, FM = WM / 16;
  static constexpr int WROW = W4 ? BK / 2 : BK;  // weight bytes per row/stage
  static constexpr int WSTRIDE = WROW + 16;
  static constexpr int XSTRIDE = BK + 16;
  static constexpr int WCPR = WROW / 16, XCPR = BK / 16;  // chunks per row
  static constexpr int WCH = BN * WCPR / NT, XCH = BM * XCPR / NT;
  static constexpr int WBYTES = BN * WSTRIDE, XBYTES = BM * XSTRIDE;
  static constexpr int STAGE = WBYTES + XBYTES;
  static_assert((BN * WCPR) % NT == 0 && (BM * XCPR) % NT == 0, "tile/threads");
  static_assert(WN % 16 == 0 && WM % 16 == 0, "wave tile");
};

template <class C, bool RAW>
__global__ void __launch_bounds__(C::NT)
gemm_tiled_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[2 * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;

  // tile order: XCD-contiguous ranges, then groups of 8 token tiles that
  // share one weight tile
  const int tiles_n = (p.N + C::BN - 1) / C::BN;
  const int tiles_m = (p.M + C::BM - 1) / C::BM;
  const int pid = xcd_remap(blockIdx.x, tiles_n * tiles_m);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int first_m = (pid / per_group) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (pid % per_group) % gsz;
  const int tn = (pid % per_group) / gsz;
  const int n0 = tn * C::BN, m0 = tm * C::BM;
  const int wn0 = (wave % C::NWN) * C::WN, wm0 = (wave / C::NWN) * C::WM;

  const int ldw = C::W4 ? p.K / 2 : p.K;
  const char *W = static_cast<const char *>(p.qw);
  const char *X = reinterpret_cast<const char *>(p.qx);

  // token scales for this lane's columns, read before the main loop
  float sxv[C::FM];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int t = m0 + wm0 + fm * 16 + r16;
    sxv[fm] = (!RAW && t < p.M) ? p.sx[t] : 0.0f;
  }

  v4i acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  v4i wreg[C::WCH], xreg[C::XCH];
  const v4i zero = {0, 0, 0, 0};

  auto load_stage = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::WCH; ++i) {
      const int c = tid + i * C::NT;
      const int row = c / C::WCPR, col = c % C::WCPR;
      const int n = n0 + row;
      const int kb = kt * C::WROW + col * 16;
      wreg[i] = (n < p.N && kb < ldw) ? ld16(W + (size_t)n * ldw + kb) : zero;
    }
#pragma unroll
    for (int i = 0; i < C::XCH; ++i) {
      const int c = tid + i * C::NT;
      const int row = c / C::XCPR, col = c % C::XCPR;
      const int t = m0 + row;
      const int kb = kt * C::BK + col * 16;
      v4i v = (t < p.M && kb < p.K) ? ld16(X + (size_t)t * p.K + kb) : zero;
      if constexpr (C::W4) v = perm_even_odd(v);
      xreg[i] = v;
    }
  };
  auto store_stage = [&](int buf) {
    char *ws = lds + buf * C::STAGE;
    char *xs = ws + C::WBYTES;
#pragma unroll
    for (int i = 0; i < C::WCH; ++i) {
      const int c = tid + i * C::NT;
      *reinterpret_cast<v4i *>(ws + (c / C::WCPR) * C::WSTRIDE + (c % C::WCPR) * 16) = wreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::XCH; ++i) {
      const int c = tid + i * C::NT;
      *reinterpret_cast<v4i *>(xs + (c / C::XCPR) * C::XSTRIDE + (c % C::XCPR) * 16) = xreg[i];
    }
  };
  auto compute = [&](int buf) {
    const char *ws = lds + buf * C::STAGE;
    const char *xs = ws + C::WBYTES;
    if constexpr (!C::W4) {
#pragma unroll
      for (int s = 0; s < C::BK / 64; ++s) {
        v4i a[C::FN], b[C::FM];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          a[fn] = ld16(ws + (wn0 + fn * 16 + r16) * C::WSTRIDE + s * 64 + g * 16);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
          b[fm] = ld16(xs + (wm0 + fm * 16 + r16) * C::XSTRIDE + s * 64 + g * 16);
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm)
            acc[fn][fm] = mfma_i8(a[fn], b[fm], acc[fn][fm]);
      }
    } else {
      // one 16-byte packed read covers k = 32g .. 32g+31 of the stage:
      // bytes 0-7 feed MFMA slot 0 and bytes 8-15 slot 1
      v4i raw[C::FN];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        raw[fn] = ld16(ws + (wn0 + fn * 16 + r16) * C::WSTRIDE + g * 16);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v4i a[C::FN], b[C::FM];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          a[fn] = unpack_w4(raw[fn][2 * s], raw[fn][2 * s + 1]);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
          b[fm] = ld16(xs + (wm0 + fm * 16 + r16) * C::XSTRIDE + g * 32 + s * 16);
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm)
            acc[fn][fm] = mfma_i8(a[fn], b[fm], acc[fn][fm]);
      }
    }
  };

  const int KT = (p.K + C::BK - 1) / C::BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_stage(kt + 1);
    compute(cur);
    if (kt + 1 < KT) store_stage(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int t = m0 + wm0 + fm * 16 + r16;
      const int nb = n0 + wn0 + fn * 16 + g * 4;
      store_quad<C::W4, RAW>(p, t, nb, acc[fn][fm], sxv[fm]);
    }
}

// ================================================================= skinny
// Decode-sized M (<= 64): the weights are streamed from HBM once, straight
// into MFMA operand registers (no LDS staging).  A block owns BN weight rows
// and all M tokens; its NW waves split K (wave w takes k-steps w, w+NW, ...
// so the block reads NW adjacent 64-byte segments of every row at a time),
// keep U steps of loads in flight, and finally add their int32 partial sums
// in LDS (integer addition: exact and order-free) before the epilogue.
template <int BN_, int MF_, int NW_, int U_, bool W4_>
struct Skinny {
  static constexpr int BN = BN_, MF = MF_, NW = NW_, U = U_;
  static constexpr bool W4 = W4_;
  static constexpr int FN = BN / 16;
  static constexpr int NT = NW * kWave;
  static constexpr int KSTEP = W4 ? 128 : 64;  // k per step per lane group
};

template <class C, bool RAW>
__global__ void __launch_bounds__(C::NT)
gemm_skinny_kernel(GemmArgs p) {
  __shared__ int red[C::FN * C::MF * kWave * 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * C::BN;
  const int ldw = C::W4 ? p.K / 2 : p.K;
  const char *W = static_cast<const char *>(p.qw);
  const char *X = reinterpret_cast<const char *>(p.qx);
  const v4i zero = {0, 0, 0, 0};

  for (int i = tid; i < C::FN * C::MF * kWave * 4; i += C::NT) red[i] = 0;

  v4i acc[C::FN][C::MF];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::MF; ++j) acc[i][j] = zero;

  // per-lane row pointers (rows past N / tokens past M read nothing)
  const char *wrow[C::FN];
  bool wok[C::FN];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const int n = n0 + fn * 16 + r16;
    wok[fn] = n < p.N;
    wrow[fn] = W + (size_t)(wok[fn] ? n : 0) * ldw + g * 16;
  }
  const char *xrow[C::MF];
  bool xok[C::MF];
#pragma unroll
  for (int fm = 0; fm < C::MF; ++fm) {
    const int t = fm * 16 + r16;
    xok[fm] = t < p.M;
    xrow[fm] = X + (size_t)(xok[fm] ? t : 0) * p.K + g * (C::W4 ? 32 : 16);
  }

  const int nsteps = p.K / C::KSTEP;
  for (int s0 = wave; s0 < nsteps; s0 += C::NW * C::U) {
    v4i wv[C::U][C::FN];
    v4i xv[C::U][C::MF][C::W4 ? 2 : 1];
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      const int s = s0 + u * C::NW;
      const bool ok = s < nsteps;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        wv[u][fn] = (ok && wok[fn]) ? ld16(wrow[fn] + (size_t)s * 64) : zero;
#pragma unroll
      for (int fm = 0; fm < C::MF; ++fm) {
        if constexpr (C::W4) {
          const bool o = ok && xok[fm];
          xv[u][fm][0] = o ? ld16(xrow[fm] + (size_t)s * 128) : zero;
          xv[u][fm][1] = o ? ld16(xrow[fm] + (size_t)s * 128 + 16) : zero;
        } else {
          xv[u][fm][0] = (ok && xok[fm]) ? ld16(xrow[fm] + (size_t)s * 64) : zero;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < C::MF; ++fm) {
          if constexpr (C::W4) {
            acc[fn][fm] = mfma_i8(unpack_w4(wv[u][fn][0], wv[u][fn][1]),
                                  perm_even_odd(xv[u][fm][0]), acc[fn][fm]);
            acc[fn][fm] = mfma_i8(unpack_w4(wv[u][fn][2], wv[u][fn][3]),
                                  perm_even_odd(xv[u][fm][1]), acc[fn][fm]);
          } else {
            acc[fn][fm] = mfma_i8(wv[u][fn], xv[u][fm][0], acc[fn][fm]);
          }
        }
    }
  }
  if constexpr (C::W4) {
    // K % 128 == 64: one last half step of 64 k, 8 packed bytes per lane
    if ((p.K % 128) != 0 && wave == (nsteps % C::NW)) {
      const size_t kb = (size_t)nsteps * 64;  // packed byte offset
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        v2i w8 = {0, 0};
        if (wok[fn])
          w8 = *reinterpret_cast<const v2i *>(wrow[fn] - g * 16 + kb + g * 8);
#pragma unroll
        for (int fm = 0; fm < C::MF; ++fm) {
          v4i x = xok[fm] ? ld16(xrow[fm] - g * 32 + (size_t)nsteps * 128 + g * 16) : zero;
          acc[fn][fm] = mfma_i8(unpack_w4(w8[0], w8[1]), perm_even_odd(x), acc[fn][fm]);
        }
      }
    }
  }

  __syncthreads();  // red[] zeroed
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
    for (int fm = 0; fm < C::MF; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        atomicAdd(&red[((fn * C::MF + fm) * kWave + lane) * 4 + r], acc[fn][fm][r]);
  __syncthreads();

  for (int pr = wave; pr < C::FN * C::MF; pr += C::NW) {
    const int fn = pr / C::MF, fm = pr % C::MF;
    v4i a;
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = red[(pr * kWave + lane) * 4 + r];
    const int t = fm * 16 + r16;
    const int nb = n0 + fn * 16 + g * 4;
    const float sxt = (!RAW && t < p.M) ? p.sx[t] : 0.0f;
    store_quad<C::W4, RAW>(p, t, nb, a, sxt);
  }
}

// ================================================================ dispatch
template <class C, bool RAW>
static hipError_t run_tiled(const GemmArgs &a, hipStream_t s) {
  const int tiles = ((a.N + C::BN - 1) / C::BN) * ((a.M + C::BM - 1) / C::BM);
  hipLaunchKernelGGL((gemm_tiled_kernel<C, RAW>), dim3(tiles), dim3(C::NT), 0,
                     s, a);
  return hipGetLastError();
}

template <class C, bool RAW>
static hipError_t run_skinny(const GemmArgs &a, hipStream_t s) {
  const int blocks = (a.N + C::BN - 1) / C::BN;
  hipLaunchKernelGGL((gemm_skinny_kernel<C, RAW>), dim3(blocks), dim3(C::NT),
                     0, s, a);
  return hipGetLastError();
}

enum PlanKind { kSkinny = 0, kTiled = 1 };
struct Plan {
  PlanKind kind;
  int mf;  // skinny: 16-token fragments
};

static Plan choose(int M, int /*N*/, int /*K*/, int /*bits*/) {
  if (M <= 64) return Plan{kSkinny, (M + 15) / 16};
  return Plan{kTiled, 0};
}

template <bool W4, bool RAW>
static hipError_t run(const GemmArgs &a, hipStream_t s) {
  const Plan pl = choose(a.M, a.N, a.K, a.bits);
  if (pl.kind == kSkinny) {
    switch (pl.mf) {
      case 1: return run_skinny<Skinny<16, 1, 8, 4, W4>, RAW>(a, s);
      case 2: return run_skinny<Skinny<16, 2, 8, 4, W4>, RAW>(a, s);
      case 3: return run_skinny<Skinny<16, 3, 8, 2, W4>, RAW>(a, s);
      default: return run_skinny<Skinny<16, 4, 8, 2, W4>, RAW>(a, s);
    }
  }
  return run_tiled<Tile<128, 128, 64, 64, W4>, RAW>(a, s);
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t s) {
  if (a.bits == 4)
    return a.raw_i32 ? run<true, true>(a, s) : run<true, false>(a, s);
  return a.raw_i32 ? run<false, true>(a, s) : run<false, false>(a, s);
}

int describe_gemm_plan(int M, int N, int K, int bits, char *buf, int len) {
  const Plan pl = choose(M, N, K, bits);
  if (pl.kind == kSkinny)
    return snprintf(buf, len, "skinny BN=16 MF=%d NW=8 U=%d W%d blocks=%d",
                    pl.mf, pl.mf <= 2 ? 4 : 2, bits, (N + 15) / 16);
  return snprintf(buf, len, "tiled BN=128 BM=128 WN=64 WM=64 BK=128 W%d tiles=%d",
                  bits, ((N + 127) / 128) * ((M + 127) / 128));
}

}  // namespace zq
