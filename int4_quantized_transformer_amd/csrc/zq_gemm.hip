// zq_gemm.hip -- INT8 x INT8 GEMM with fused dequantization for gfx950.
//
// ZeroQuant summary page, Sec. 3.4 "Quantization-Optimized Transformer
// Kernels" (paper Sec. 4.3, App. D): an INT8 GEMM whose epilogue turns the
// INT32 accumulator into fp16 with the per-token activation scale and the
// per-group weight scale (read before the main loop ends), so that no
// separate dequantization kernel runs; the tiling is picked per token count
// (throughput-oriented for large batches, bandwidth-oriented for small).
//
// Kernels: gemm_tiled_kernel (v_mfma_i32_32x32x32_i8; more than 64 tokens,
// and W8 with 33..64 tokens over N >= 8192), gemm_stream_kernel (per-wave
// LDS rings of 1, 16, 32 or 64 token rows; up to 64 tokens, even N),
// gemm_skinny_kernel (up to 64 tokens, odd N) and gemm_gemv_kernel
// (v_dot4_i32_i8; one token).  In the v_mfma_i32_16x16x64_i8 kernels
// (streaming, skinny) the weight tile is the MFMA "A" operand (rows =
// output features n) and the activation tile the "B" operand (columns =
// tokens t), so each lane ends with 4 consecutive n of one token:
// y[t][n..n+3] is one 8-byte store.  Within one MFMA the
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
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "zq_internal.h"

#define ZQ_GPTR(p) ((__attribute__((address_space(1))) void *)(p))
#define ZQ_LPTR(p) ((__attribute__((address_space(3))) void *)(p))

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

// s_waitcnt with vmcnt = N and no wait on the other counters (gfx9
// encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) |
                             ((N >> 4) << 14));
}

// ---------------------------------------------------------------- epilogue
// Output columns of one fragment row: n = nb .. nb+3.  The group scale and
// the bias are fetched once per fragment, before the main loop (their
// latency hides behind it), and reused for every token of the tile.  All
// loads are unconditional with clamped indices so that no wait is needed
// until the epilogue uses them.
struct QuadCol {
  float sw[4];
  half_t b[4];
};

__device__ __forceinline__ QuadCol load_quad_col(const GemmArgs &p, int nb) {
  QuadCol c;
  const int n = nb < p.N ? nb : p.N - 1;
  const int g0 = n / p.G;
  const int rem = n - g0 * p.G;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    // group of column n + r: g0 + (rem + r) / G, which for G >= 4 is
    // g0 or g0 + 1; clamp to the last column
    int gi;
    if (p.G >= 4) {
      gi = g0 + (rem + r >= p.G ? 1 : 0);
    } else {
      gi = (n + r) / p.G;
    }
    const int last = (p.N - 1) / p.G;
    c.sw[r] = p.sw[gi < last ? gi : last];
  }
  if (p.bias) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c.b[r] = p.bias[n + r < p.N ? n + r : p.N - 1];
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) c.b[r] = (half_t)0.0f;
  }
  return c;
}

// y = fp16(act(float(acc) * (sx[t] * sw[n / G]) + bias[n])), or the raw
// int32 accumulator.  Lane holds n = nb .. nb+3 of token t.  FACC: acc holds
// fp32 sums (the fp16-activation GEMM) as raw bits.
template <bool W4, bool RAW, bool FACC = false>
__device__ __forceinline__ void store_quad(const GemmArgs &p, int t, int nb,
                                           v4i acc, float sxt,
                                           const QuadCol &c) {
  if (t >= p.M || nb >= p.N) return;
  if constexpr (W4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] >>= 4;
  }
  const bool full = nb + 3 < p.N && (p.N & 3) == 0;
  if constexpr (RAW) {
    int32_t *o = static_cast<int32_t *>(p.out) + (size_t)t * p.N + nb;
    if (full) {
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
      const float sc = sxt * c.sw[r];
      // the element is copied out first: this compiler's __builtin_bit_cast
      // of a vector element (acc[r]) reads element 0
      const int ai = acc[r];
      const float a = FACC ? __builtin_bit_cast(float, ai) : (float)ai;
      h[r] = p.act == ZQ_ACT_GELU ? gelu_half(a, sc, c.b[r])
                                  : fma_half(a, sc, c.b[r]);
    }
    half_t *o = static_cast<half_t *>(p.out) + (size_t)t * p.N + nb;
    if (full) {
      *reinterpret_cast<half4 *>(o) = h;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nb + r < p.N) o[r] = h[r];
    }
  }
}

// =================================================================== tiled
// Prefill-sized M.  v_mfma_i32_32x32x32_i8 (on gfx950 it sustains twice the
// integer rate of the 16x16x64 form): lane l holds row l%32 of a 32x32
// operand block and 16 k-bytes chosen by its lane half h = l/32; the result
// lane l holds token t = l%32 and outputs n = 8q + 4h + (0..3), q = 0..3.
//
// Block tile BN (n) x BM (t), k in stages of KB = 128 activation bytes
// (64 packed W4 bytes), or KB = 64 for W8 (half the bytes per stage, so
// twice the stages fit in LDS and more of them are in flight).  Operands travel global -> LDS directly
// (global_load_lds_dwordx4: each lane's 16 bytes land at a wave-contiguous
// LDS address, no register staging) through an S-stage ring; while stage k
// is multiplied, stages k+1 .. k+S-1 are in flight.  One barrier per stage:
// a wave waits for its own copies of stage k (vmcnt), the barrier makes all
// copies visible, and only then is stage k+S-1 issued into the slot that
// stage k-1 used.
//
// LDS rows are unpadded (128 B, or 64 B for packed W4) and their 16-byte
// chunks are XOR-swizzled so that the 16-byte fragment reads of 8
// consecutive rows (one LDS cycle) hit 8 different bank groups:
//   128-byte rows: slot = chunk ^ ((row >> 1) & 7)
//    64-byte rows: slot = chunk ^ ((row >> 2) & 3)

__device__ __forceinline__ v16i mfma32_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

template <class C>
__device__ __forceinline__ void issue_stage(const GemmArgs &p, const char *W,
                                            const char *X, int ldw, int n0,
                                            int m0, int kt, char *stage,
                                            int wave, int lane) {
#pragma unroll
  for (int j = 0; j < C::IW; ++j) {
    const CopyAddr c = tile_w_copy<C>(wave * C::IW + j, lane, n0, kt, p.N, ldw);
    __builtin_amdgcn_global_load_lds(ZQ_GPTR(W + c.goff), ZQ_LPTR(stage + c.lds),
                                     16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < C::IX; ++j) {
    const CopyAddr c = tile_x_copy<C>(wave * C::IX + j, lane, m0, kt, p.M, p.K);
    __builtin_amdgcn_global_load_lds(ZQ_GPTR(X + c.goff), ZQ_LPTR(stage + c.lds),
                                     16, 0, 0);
  }
}

// Wait until at most `left` stages of this wave's copies are in flight
// (left <= S - 2; each stage is P copies per wave, completed in order).
template <class C, int L = C::S - 2>
__device__ __forceinline__ void wait_stages(int left) {
  constexpr int P = C::IW + C::IX;
  if constexpr (L > 0) {
    if (left >= L) {
      wait_vmcnt<L * P>();
      return;
    }
    wait_stages<C, L - 1>(left);
  } else {
    wait_vmcnt<0>();
  }
}

// Operand fragments of one MFMA k-step (32 k): weights a[FN] (for W4 the
// packed source, unpacked at use), activations b[FM].
template <class C>
struct Frag {
  v4i a[C::FN];
  v4i b[C::FM];
};

// Full stage, k-step s (0 .. KS-1), lane half h.
//   W8: weight and activation chunk 2s + h (k = 32s + 16h) of the stage's
//       KB-byte rows.
//   W4: lane half h takes k = 64h + 16s: packed chunk 2h (s = 0, 1) or
//       2h + 1 (s = 2, 3), read once per pair into raw0 / raw1, and
//       activation chunk 4h + s.
template <class C>
__device__ __forceinline__ void fetch(const char *ws, const char *xs, int s,
                                      int wn0, int wm0, int r32, int h,
                                      Frag<C> &f, v4i (&raw)[2][C::FN]) {
  const int x7 = sw128(r32);
  if constexpr (C::A16) {
    // activations: 8 halves (chunk 2s + h of the 128-byte row, k = 16s + 8h);
    // weights: the matching 8 codes, half h of chunk s of the 64-byte row
    const int c = wswz<C::XROW>(2 * s + h, r32);
    const int cw = s ^ sw64(r32);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const v2i w = *reinterpret_cast<const v2i *>(
          ws + (wn0 + fn * 32 + r32) * 64 + (cw << 4) + 8 * h);
      f.a[fn] = v4i{w[0], w[1], 0, 0};
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
      f.b[fm] = ld16(xs + (wm0 + fm * 32 + r32) * C::XROW + (c << 4));
  } else if constexpr (!C::W4) {
    // rows of XROW bytes; the swizzle depends on the row's low bits only,
    // which r32 shares with every fragment row
    const int c = wswz<C::XROW>(2 * s + h, r32);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
      f.a[fn] = ld16(ws + (wn0 + fn * 32 + r32) * C::XROW + (c << 4));
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
      f.b[fm] = ld16(xs + (wm0 + fm * 32 + r32) * C::XROW + (c << 4));
  } else {
    const int w4 = sw64(r32);
    if (s == 0 || s == 2) {
      const int pc = 2 * h + (s >> 1);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        raw[s >> 1][fn] = ld16(ws + (wn0 + fn * 32 + r32) * 64 + ((pc ^ w4) << 4));
    }
    const int c = 4 * h + s;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
      f.b[fm] = ld16(xs + (wm0 + fm * 32 + r32) * 128 + ((c ^ x7) << 4));
  }
}

// Eight INT8 codes (two words) as eight fp16 values, exactly: with the
// sign bit flipped a byte is u = q + 128; placed under the fp16 exponent of
// 1024 (bits 0x64uu) it reads 1024 + u, and 1024 + u - 1152 = q.  The
// halves are assembled with shifts and masks.
__device__ __forceinline__ v4i i8x8_to_f16x8(int w0, int w1) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 bias = {(half_t)1152.0f, (half_t)1152.0f};
  const uint32_t u[2] = {(uint32_t)w0 ^ 0x80808080u, (uint32_t)w1 ^ 0x80808080u};
  v4i r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // bytes 0, 1 -> halves of word 2i; bytes 2, 3 -> halves of word 2i + 1
    const uint32_t lo = (u[i] & 0xFFu) | ((u[i] << 8) & 0xFF0000u) | 0x64006400u;
    const uint32_t hi = ((u[i] >> 16) & 0xFFu) | ((u[i] >> 8) & 0xFF0000u) | 0x64006400u;
    r[2 * i] = __builtin_bit_cast(int, __builtin_bit_cast(h2, lo) - bias);
    r[2 * i + 1] = __builtin_bit_cast(int, __builtin_bit_cast(h2, hi) - bias);
  }
  return r;
}

template <class C>
__device__ __forceinline__ void mma(const Frag<C> &f, int s,
                                    const v4i (&raw)[2][C::FN],
                                    v16i (&acc)[C::FN][C::FM]) {
  if constexpr (C::A16) {
    typedef float v16f __attribute__((ext_vector_type(16)));
    v4i a[C::FN];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) a[fn] = i8x8_to_f16x8(f.a[fn][0], f.a[fn][1]);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
        acc[fn][fm] = __builtin_bit_cast(
            v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(
                      __builtin_bit_cast(half8, a[fn]),
                      __builtin_bit_cast(half8, f.b[fm]),
                      __builtin_bit_cast(v16f, acc[fn][fm]), 0, 0, 0));
    return;
  }
  v4i a[C::FN], b[C::FM];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    if constexpr (C::W4) {
      const v4i &rw = raw[s >> 1][fn];
      a[fn] = unpack_w4(rw[2 * (s & 1)], rw[2 * (s & 1) + 1]);
    } else {
      a[fn] = f.a[fn];
    }
  }
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
    b[fm] = C::W4 ? perm_even_odd(f.b[fm]) : f.b[fm];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
      acc[fn][fm] = mfma32_i8(a[fn], b[fm], acc[fn][fm]);
}

// lgkmcnt(N), no wait on the other counters.
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (N << 8) | (0x3 << 14));
}

// 64-k tail stage, k-step s (0, 1): k = 32s + 16h.  W8: chunk 2s + h.
// W4: packed bytes 16s + 8h .. +7 (chunk s, half h), activation chunk
// 2s + h.  Fetched and multiplied without overlap (it happens once).
template <class C>
__device__ __forceinline__ void tail_stage(const char *ws, const char *xs,
                                           int wn0, int wm0, int r32, int h,
                                           v16i (&acc)[C::FN][C::FM]) {
  const int x7 = sw128(r32);
  const int w4 = sw64(r32);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v4i a[C::FN], b[C::FM];
    const int c = 2 * s + h;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      if constexpr (C::W4) {
        const v2i w = *reinterpret_cast<const v2i *>(
            ws + (wn0 + fn * 32 + r32) * 64 + ((s ^ w4) << 4) + h * 8);
        a[fn] = unpack_w4(w[0], w[1]);
      } else {
        a[fn] = ld16(ws + (wn0 + fn * 32 + r32) * 128 + ((c ^ x7) << 4));
      }
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const v4i x = ld16(xs + (wm0 + fm * 32 + r32) * 128 + ((c ^ x7) << 4));
      b[fm] = C::W4 ? perm_even_odd(x) : x;
    }
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
        acc[fn][fm] = mfma32_i8(a[fn], b[fm], acc[fn][fm]);
  }
}

// Main loop schedule (S LDS slots; stage j is copied into slot j % S):
//   prologue: copy stages 0 .. S-1, wait for stage 0, barrier, read the
//             fragments of (stage 0, k-step 0).
//   stage kt, k-step s < KS-1: read fragments of k-step s+1 into the
//             other register set, then issue the MFMAs of k-step s (the
//             reads complete under the MFMAs).
//   k-step KS-1: wait for stage kt+1's copies and for this wave's LDS reads,
//             barrier (now every wave is done with slot kt % S and stage
//             kt+1 is visible), copy stage kt+S into slot kt % S, read
//             fragments of (stage kt+1, k-step 0), MFMAs of k-step KS-1.
// Staged epilogue of the tiled kernel.  The fp16 tile goes through LDS so
// that every global store writes whole row segments with 16 bytes per lane.
// Layout: row t of the tile holds BN halves; its 16-byte chunks are
// XOR-swizzled by (t & (SW-1)), SW the largest power of two dividing the
// chunk count (at most 16), so that the 8-byte writes of consecutive rows
// spread over the banks.
template <class C>
struct StageLayout {
  static constexpr int RB = C::BN * 2;  // bytes per tile row
  static constexpr int CPR = C::BN / 8;  // 16-byte chunks per tile row
  static constexpr int SW = (CPR % 16 == 0) ? 16 : (CPR % 8 == 0) ? 8 : 4;
};

template <class C, bool GELU, bool BIAS>
__device__ __forceinline__ void stage_epilogue(
    const GemmArgs &p, char *lds, const v16i (&acc)[C::FN][C::FM],
    const float *sx_l, const half_t *bias_l, const float (&swv)[C::FN],
    int wn0, int wm0, int r32, int h) {
  using S = StageLayout<C>;
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int tl = wm0 + fm * 32 + r32;
      const float sc = C::A16 ? swv[fn] : sx_l[tl] * swv[fn];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = wn0 + fn * 32 + 8 * q + 4 * h;  // tile column
        half4 bb = {(half_t)0.0f, (half_t)0.0f, (half_t)0.0f, (half_t)0.0f};
        if constexpr (BIAS) bb = *reinterpret_cast<const half4 *>(bias_l + cl);
        float av[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int a = acc[fn][fm][4 * q + r];
          if constexpr (C::W4) a >>= 4;
          av[r] = C::A16 ? __builtin_bit_cast(float, a) : (float)a;
        }
        half4 hv;
        if constexpr (GELU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) hv[r] = gelu_half(av[r], sc, bb[r]);
        } else {
          typedef uint32_t u2 __attribute__((ext_vector_type(2)));
          const u2 b2 = __builtin_bit_cast(u2, bb);
          const u2 y2 = {fma_half2(av[0], av[1], sc, b2[0]),
                         fma_half2(av[2], av[3], sc, b2[1])};
          hv = __builtin_bit_cast(half4, y2);
        }
        const int chunk = (wn0 + fn * 32) / 8 + q;
        *reinterpret_cast<half4 *>(lds + tl * S::RB +
                                   ((chunk ^ (tl & (S::SW - 1))) << 4) + h * 8) = hv;
      }
    }
}

template <class C>
__device__ __forceinline__ void store_staged_tile(const GemmArgs &p,
                                                  const char *lds, int n0,
                                                  int m0, int tid) {
  using S = StageLayout<C>;
  const bool vec = (p.N & 7) == 0 && (((uintptr_t)p.out) & 15) == 0;
  half_t *Y = static_cast<half_t *>(p.out);
  for (int i = tid; i < C::BM * S::CPR; i += C::NT) {
    const int row = i / S::CPR, c = i % S::CPR;
    const int t = m0 + row, n = n0 + c * 8;
    if (t >= p.M || n >= p.N) continue;
    const v4i v = ld16(lds + row * S::RB + ((c ^ (row & (S::SW - 1))) << 4));
    half_t *o = Y + (size_t)t * p.N + n;
    if (vec && n + 8 <= p.N) {
      *reinterpret_cast<v4i *>(o) = v;
    } else {
      const half8 hv = __builtin_bit_cast(half8, v);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < p.N) o[e] = hv[e];
    }
  }
}

// Everything a tile needs after its main loop.
template <class C>
struct TileCtx {
  int n0, m0, tn, tm, tiles_n, tiles_m;
  int wave, lane, r32, h, wn0, wm0;
  bool g32, bias_lds;
  float swv[C::FN];
  const half_t *bias_l;  // the tile's bias (LDS aux), when bias_lds
  const float *sx_l;     // the tile's token scales (LDS aux)
};

// Tile setup, epilogue operand prefetch and the main loop: on return acc
// holds the tile's int32 sums (16*sum for W4) and every wave is past its
// last LDS operand read (LDS may be reused after a barrier).
template <class C, bool RAW>
__device__ __forceinline__ void tile_mainloop(const GemmArgs &p, char *lds,
                                              TileCtx<C> &x,
                                              v16i (&acc)[C::FN][C::FM]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, h = lane >> 5;
  x.wave = wave;
  x.lane = lane;
  x.r32 = r32;
  x.h = h;

  // tile order: XCD-contiguous ranges, then groups of 4 token tiles that
  // share one weight tile (an XCD's 32 concurrent tiles: 8 weight tiles x 4
  // token tiles, fewer operand bytes into its L2 than 4 x 8 at the prefill
  // shapes)
  const int tiles_n = (p.N + C::BN - 1) / C::BN;
  const int tiles_m = (p.M + C::BM - 1) / C::BM;
  const int pid = xcd_remap(blockIdx.x, tiles_n * tiles_m);
  int tm, tn;
  grouped_tile<kTileGroup>(pid, tiles_m, tiles_n, tm, tn);
  const int n0 = tn * C::BN, m0 = tm * C::BM;
  const int wn0 = (wave % C::NWN) * C::WN, wm0 = (wave / C::NWN) * C::WM;
  x.n0 = n0;
  x.m0 = m0;
  x.tn = tn;
  x.tm = tm;
  x.tiles_n = tiles_n;
  x.tiles_m = tiles_m;
  x.wn0 = wn0;
  x.wm0 = wm0;

  const int ldw = C::W4 ? p.K / 2 : p.K;
  const char *W = static_cast<const char *>(p.qw);
  const char *X = reinterpret_cast<const char *>(p.qx);

  // Epilogue operands are fetched before the main loop so that their
  // latency hides behind it (scales read before the multiplication ends).
  // The tile's bias (BN halves) and token scales (BM floats) are copied by
  // wave 0 straight into LDS, ahead of its stage-0 copies, so the stage-0
  // wait and barrier also cover them.  Group scale: when 32 | G every
  // 32-row weight fragment lies in one group, so one register per fragment.
  char *aux = lds + C::S * C::STAGE;
  x.g32 = (p.G & 31) == 0;
  x.bias_lds = p.bias && (p.N % 2 == 0) && (((uintptr_t)p.bias & 3) == 0);
  if constexpr (!RAW) {
    if (wave == 0) {
      if (x.bias_lds) {
#pragma unroll
        for (int j = 0; j < C::AUX_BIAS / 256; ++j) {
          int n = n0 + 2 * (lane + 64 * j);
          n = n < p.N ? n : p.N - 2;
          __builtin_amdgcn_global_load_lds(ZQ_GPTR(p.bias + n),
                                           ZQ_LPTR(aux + j * 256), 4, 0, 0);
        }
      }
      if constexpr (!C::A16) {  // fp16 activations carry no token scale
#pragma unroll
        for (int j = 0; j < C::AUX_SX / 256; ++j) {
          int t = m0 + lane + 64 * j;
          t = t < p.M ? t : p.M - 1;
          __builtin_amdgcn_global_load_lds(ZQ_GPTR(p.sx + t),
                                           ZQ_LPTR(aux + C::AUX_BIAS + j * 256),
                                           4, 0, 0);
        }
      }
    }
    const int lastg = (p.N - 1) / p.G;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int gi = (n0 + wn0 + fn * 32) / p.G;
      x.swv[fn] = x.g32 ? p.sw[gi < lastg ? gi : lastg] : 0.0f;
    }
  }
  x.bias_l = reinterpret_cast<const half_t *>(aux);
  x.sx_l = reinterpret_cast<const float *>(aux + C::AUX_BIAS);

#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = v16i{};

  // A split over K (grid y > 1) gives this workgroup the stages [kbase,
  // kbase + KT); the launcher makes K a multiple of the slices' stages, so
  // there is no half tail then.
  const int KT = ((p.K + C::KPS - 1) / C::KPS) / (int)gridDim.y;
  const int kbase = (int)blockIdx.y * KT;
  const bool half_tail = (p.K % C::KPS) != 0;   // last stage holds half
  const int KTF = KT - (half_tail ? 1 : 0);      // stages with 128 k

  const int npro = KT < C::S ? KT : C::S;
  for (int j = 0; j < npro; ++j)
    issue_stage<C>(p, W, X, ldw, n0, m0, kbase + j, lds + j * C::STAGE, wave,
                   lane);
  wait_stages<C>(npro - 1);
  __builtin_amdgcn_s_barrier();

  Frag<C> f0, f1;
  v4i raw[2][C::FN];
  if (KTF > 0) fetch<C>(lds, lds + C::WBYTES, 0, wn0, wm0, r32, h, f0, raw);
  // Scalar loads (the group scales above) share the LDS counter and return
  // out of order: while one is pending every LDS wait in the loop would
  // have to be lgkmcnt(0).  Complete them here, once.
  wait_lgkmcnt<0>();
  __builtin_amdgcn_sched_barrier(0);

  // sched_barrier(0) keeps the phases in this order (the scheduler would
  // otherwise hoist the barrier above the MFMAs of k-step 2).
  for (int kt = 0; kt < KTF; ++kt) {
    char *ws = lds + (kt % C::S) * C::STAGE;
    const char *xs = ws + C::WBYTES;
    fetch<C>(ws, xs, 1, wn0, wm0, r32, h, f1, raw);
    mma<C>(f0, 0, raw, acc);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (C::KS == 4) {
      fetch<C>(ws, xs, 2, wn0, wm0, r32, h, f0, raw);
      mma<C>(f1, 1, raw, acc);
      __builtin_amdgcn_sched_barrier(0);
      fetch<C>(ws, xs, 3, wn0, wm0, r32, h, f1, raw);
      mma<C>(f0, 2, raw, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    // last k-step (KS - 1, held in f1): stage boundary
    wait_stages<C>(max(0, min(C::S - 2, KT - 2 - kt)));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): own LDS reads done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (kt + C::S < KT)
      issue_stage<C>(p, W, X, ldw, n0, m0, kbase + kt + C::S, ws, wave, lane);
    {
      // unconditional (after the last stage it reads a stale slot, in
      // bounds, and the fragments go unused): a conditional read here
      // makes the compiler wait for every LDS read at the loop head
      char *wn = lds + ((kt + 1) % C::S) * C::STAGE;
      fetch<C>(wn, wn + C::WBYTES, 0, wn0, wm0, r32, h, f0, raw);
    }
    mma<C>(f1, C::KS - 1, raw, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (C::KB == 128 && !C::A16) if (half_tail) {
    const char *ws = lds + ((KT - 1) % C::S) * C::STAGE;
    tail_stage<C>(ws, ws + C::WBYTES, wn0, wm0, r32, h, acc);
  }
}

template <class C, bool RAW>
__global__ void __launch_bounds__(C::NT)
gemm_tiled_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  // split over K: each slice writes its raw sums to its own M x N plane
  if constexpr (RAW)
    p.out = static_cast<int32_t *>(p.out) + (size_t)blockIdx.y * p.M * p.N;
  TileCtx<C> x;
  v16i acc[C::FN][C::FM];
  tile_mainloop<C, RAW>(p, lds, x, acc);
  const int r32 = x.r32, h = x.h, wn0 = x.wn0, wm0 = x.wm0;
  const int n0 = x.n0, m0 = x.m0;

  if constexpr (!RAW && C::BM * C::BN * 2 <= C::S * C::STAGE && C::BN >= 64) {
    if (x.g32 && (x.bias_lds || !p.bias)) {
      __syncthreads();  // every wave is done reading the operand stages
      // the activation and the bias are uniform: one straight-line variant
      // each, so that independent elements interleave
      if (p.act == ZQ_ACT_GELU) {
        if (p.bias) stage_epilogue<C, true, true>(p, lds, acc, x.sx_l, x.bias_l, x.swv, wn0, wm0, r32, h);
        else stage_epilogue<C, true, false>(p, lds, acc, x.sx_l, x.bias_l, x.swv, wn0, wm0, r32, h);
      } else {
        if (p.bias) stage_epilogue<C, false, true>(p, lds, acc, x.sx_l, x.bias_l, x.swv, wn0, wm0, r32, h);
        else stage_epilogue<C, false, false>(p, lds, acc, x.sx_l, x.bias_l, x.swv, wn0, wm0, r32, h);
      }
      __syncthreads();
      store_staged_tile<C>(p, lds, n0, m0, threadIdx.x);
      return;
    }
  }

#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int t = m0 + wm0 + fm * 32 + r32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nb = n0 + wn0 + fn * 32 + 8 * q + 4 * h;
        const v4i a = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1],
                       acc[fn][fm][4 * q + 2], acc[fn][fm][4 * q + 3]};
        QuadCol qc;
        float sxt = 0.0f;
        if constexpr (!RAW) {
          qc = load_quad_col(p, nb);
          sxt = C::A16 ? 1.0f : p.sx[t < p.M ? t : p.M - 1];
        }
        store_quad<C::W4, RAW, C::A16>(p, t, nb, a, sxt, qc);
      }
    }
}

// ============================================================== ping-pong
// Prefill GEMM with packed W4 weights over wide N (the GPT-NeoX-20B FFN1
// shape): a persistent kernel, one workgroup per compute unit looping over
// 256 x 256 tiles, with the operand copies forming one continuous ring
// across tile boundaries (the next tile's first stages are in flight while
// a tile's epilogue runs).  The LDS layout and the fragment / MFMA helpers
// are those of gemm_tiled_kernel.
//
// Epilogue operands of each tile (bias of its columns, scales of its tokens,
// the group scale of each 32-column fragment) travel into one of two LDS
// buffers with the tile's first stage (before its operand copies, so the
// wait for that stage covers them); the fp16 (or int32) results are stored
// straight from registers, each lane writing 4 consecutive outputs of one
// token.


template <class C>
__device__ __forceinline__ void persist_aux_copy(const GemmArgs &p, char *ab,
                                                 int n0, int m0, int wave,
                                                 int lane) {
  using A = PAux<C>;
  for (int c = wave; c < A::NCOPY; c += C::NWAVES) {
    const AuxElem a = persist_aux_elem<C>(c * 64 + lane, n0, m0, p.M, p.G);
    const void *src = p.qw;                    // padding lanes: any dword
    if (a.src == kAuxBias)                     // without a bias: unused
      src = p.bias ? (const void *)(reinterpret_cast<const int *>(p.bias) + a.index)
                   : (const void *)p.sx;
    else if (a.src == kAuxSx)
      src = p.sx + a.index;
    else if (a.src == kAuxSw)
      src = p.sw + a.index;
    __builtin_amdgcn_global_load_lds(ZQ_GPTR(src), ZQ_LPTR(ab + c * 256), 4,
                                     0, 0);
  }
}

template <class C, bool RAW>
__device__ __forceinline__ void persist_epilogue(
    const GemmArgs &p, const char *ab, const v16i (&acc)[C::FN][C::FM],
    int n0, int m0, int wn0, int wm0, int r32, int h) {
  using A = PAux<C>;
  const half_t *bias_l = reinterpret_cast<const half_t *>(ab);
  const float *sx_l = reinterpret_cast<const float *>(ab + A::BIAS);
  const float *sw_l = reinterpret_cast<const float *>(ab + A::BIAS + A::SX);
  float swv[C::FN];
  if constexpr (!RAW) {
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) swv[fn] = sw_l[(wn0 + fn * 32) / 32];
  }
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int tl = wm0 + fm * 32 + r32;
    const int t = m0 + tl;
    const bool tok = t < p.M;
    float sxt = 0.0f;
    if constexpr (!RAW) sxt = sx_l[tl];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = wn0 + fn * 32 + 8 * q + 4 * h;  // tile column
        int a[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] = acc[fn][fm][4 * q + r];
          if constexpr (C::W4) a[r] >>= 4;
        }
        if constexpr (RAW) {
          int32_t *o = static_cast<int32_t *>(p.out) + (size_t)t * p.N + n0 + cl;
          if (tok) *reinterpret_cast<v4i *>(o) = v4i{a[0], a[1], a[2], a[3]};
        } else {
          const float sc = sxt * swv[fn];
          half4 bb = {(half_t)0.0f, (half_t)0.0f, (half_t)0.0f, (half_t)0.0f};
          if (p.bias) bb = *reinterpret_cast<const half4 *>(bias_l + cl);
          half4 hv;
          if (p.act == ZQ_ACT_GELU) {
#pragma unroll
            for (int r = 0; r < 4; ++r) hv[r] = gelu_half((float)a[r], sc, bb[r]);
          } else {
            typedef uint32_t u2 __attribute__((ext_vector_type(2)));
            const u2 b2 = __builtin_bit_cast(u2, bb);
            const u2 y2 = {fma_half2((float)a[0], (float)a[1], sc, b2[0]),
                           fma_half2((float)a[2], (float)a[3], sc, b2[1])};
            hv = __builtin_bit_cast(half4, y2);
          }
          half_t *o = static_cast<half_t *>(p.out) + (size_t)t * p.N + n0 + cl;
          if (tok) *reinterpret_cast<half4 *>(o) = hv;
        }
      }
    }
  }
}

// The two wave groups of a workgroup alternate between memory and compute: in every barrier-delimited slot one group
// reads a whole stage of operand fragments from LDS into registers (and,
// for group A, issues the global -> LDS copies of a later stage) while the
// other group runs that stage's MFMAs back to back from registers.  Waves
// w and w + 4 share a SIMD and belong to different groups, so each SIMD
// always has one wave feeding the matrix core.  Block tile 256 x 256; group
// A owns tokens 0..127 of the tile, group B tokens 128..255; each wave 64
// outputs x 128 tokens.
//
// Slot schedule (g = global stage): slot 2g: A reads stage g and issues
// the copies of stage g + S - 1 (into the slot of stage g - 1, which both
// groups have read), B computes stage g - 1; slot 2g + 1: A computes stage
// g, B reads stage g.  A waits for its copies of stage g + 1 at the end of
// slot 2g + 1, before the barrier after which both groups may read it.
template <class C>
__device__ __forceinline__ void pp_read(const char *ws, int wn0, int wm0,
                                        int r32, int h, Frag<C> (&f)[C::KS],
                                        v4i (&raw)[2][C::FN]) {
#pragma unroll
  for (int s = 0; s < C::KS; ++s)
    fetch<C>(ws, ws + C::WBYTES, s, wn0, wm0, r32, h, f[s], raw);
}

template <class C>
__device__ __forceinline__ void pp_compute(const Frag<C> (&f)[C::KS],
                                           const v4i (&raw)[2][C::FN],
                                           v16i (&acc)[C::FN][C::FM]) {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads
#pragma unroll
  for (int s = 0; s < C::KS; ++s) mma<C>(f[s], s, raw, acc);
}

template <class C, bool RAW>
__global__ void __launch_bounds__(C::NT)
gemm_pingpong_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  static_assert(C::NWAVES == 8 && C::NWN == 4 && C::NWM == 2, "ping-pong");
  using A = PAux<C>;
  __shared__ __attribute__((aligned(1024))) char lds[A::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const bool grp_a = wave < 4;
  const int wn0 = (wave % C::NWN) * C::WN, wm0 = (wave / C::NWN) * C::WM;
  char *aux = lds + C::S * C::STAGE;

  const int G = (int)gridDim.x;
  const int ntiles = tiles_m * tiles_n;
  const int slot = xcd_remap(blockIdx.x, G);
  const int mine = (ntiles - slot + G - 1) / G;
  const int KT = p.K / C::KPS;
  const int total = mine * KT;
  const int ldw = C::W4 ? p.K / 2 : p.K;
  const char *W = static_cast<const char *>(p.qw);
  const char *X = reinterpret_cast<const char *>(p.qx);

  // group A issues every copy of a stage: its own share and that of the
  // group-B wave on the same SIMD
  auto issue = [&](int g) {
    const int i = g / KT, kt = g - i * KT;
    int tm, tn;
    persist_tile(slot + i * G, tiles_m, tiles_n, tm, tn);
    char *dst = lds + (g % C::S) * C::STAGE;
    if constexpr (!RAW)
      if (kt == 0) {
        persist_aux_copy<C>(p, aux + (i & 1) * A::BYTES, tn * C::BN, tm * C::BM,
                            wave, lane);
        persist_aux_copy<C>(p, aux + (i & 1) * A::BYTES, tn * C::BN, tm * C::BM,
                            wave + 4, lane);
      }
    issue_stage<C>(p, W, X, ldw, tn * C::BN, tm * C::BM, kt, dst, wave, lane);
    issue_stage<C>(p, W, X, ldw, tn * C::BN, tm * C::BM, kt, dst, wave + 4,
                   lane);
  };
  constexpr int P2 = 2 * (C::IW + C::IX);  // operand copies per A wave per stage

  v16i acc[C::FN][C::FM];
  Frag<C> f[C::KS];
  v4i raw[2][C::FN];
  auto zero = [&]() {
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j) acc[i][j] = v16i{};
  };
  auto epilogue = [&](int itile) {
    int tm, tn;
    persist_tile(slot + itile * G, tiles_m, tiles_n, tm, tn);
    persist_epilogue<C, RAW>(p, aux + (itile & 1) * A::BYTES, acc, tn * C::BN,
                             tm * C::BM, wn0, wm0, r32, h);
  };

  if (grp_a) {
    const int npro = total < C::S - 1 ? total : C::S - 1;
    for (int g = 0; g < npro; ++g) issue(g);
    // stage 0 landed: at most the later prologue stages outstanding
    if (npro >= 3) wait_vmcnt<2 * P2>();
    else if (npro == 2) wait_vmcnt<P2>();
    else wait_vmcnt<0>();
  }
  __builtin_amdgcn_s_barrier();

  if (grp_a) {
    int g = 0;
    auto stage = [&](bool last, int itile) {
      // slot 2g: read stage g, issue stage g + S - 1
      pp_read<C>(lds + (g % C::S) * C::STAGE, wn0, wm0, r32, h, f, raw);
      if (g + C::S - 1 < total) issue(g + C::S - 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // slot 2g + 1: compute stage g; stage g + 1 must land before the
      // barrier (outstanding: the stages after it, S - 2 of them at most)
      pp_compute<C>(f, raw, acc);
      if (last) epilogue(itile);
      const int later = min(C::S - 2, total - 2 - g);
      if (later >= 2) wait_vmcnt<2 * P2>();
      else if (later == 1) wait_vmcnt<P2>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      ++g;
    };
    for (int itile = 0; itile < mine; ++itile) {
      zero();
      for (int kt = 0; kt < KT - 1; ++kt) stage(false, itile);
      stage(true, itile);
    }
  } else {
    int g = 0;
    auto read = [&]() {
      // slot 2g + 1: read stage g; the reads complete before the barrier,
      // after which group A may issue copies into this slot
      pp_read<C>(lds + (g % C::S) * C::STAGE, wn0, wm0, r32, h, f, raw);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      ++g;
    };
    for (int itile = 0; itile < mine; ++itile) {
      // slot 2g of the tile's first stage: finish the previous tile
      if (itile > 0) {
        pp_compute<C>(f, raw, acc);
        epilogue(itile - 1);
      }
      zero();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read();
      for (int kt = 1; kt < KT; ++kt) {
        // slot 2g: compute stage g - 1
        pp_compute<C>(f, raw, acc);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read();
      }
    }
    if (mine > 0) {
      pp_compute<C>(f, raw, acc);
      epilogue(mine - 1);
    }
  }
}

// ================================================================= skinny
// Decode-sized M (<= 64; chosen for odd N, where the streaming rings do not
// apply, or when forced): the weights are streamed from HBM once, straight
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
    const float sxt = RAW ? 0.0f : p.sx[t < p.M ? t : p.M - 1];
    QuadCol qc;
    if constexpr (!RAW) qc = load_quad_col(p, nb);
    store_quad<C::W4, RAW>(p, t, nb, a, sxt, qc);
  }
}

// =============================================================== streaming
// Decode-sized M (at most 64 tokens): the weight matrix is nearly all of the
// bytes and must stream from HBM at full rate, which takes many bytes in
// flight per compute unit.  Register-staged loads cannot hold enough of
// them, so every wave runs its own ring of D LDS slots fed by
// global_load_lds and waits on its own vmcnt only (no barrier per chunk).
//
// A row block is BN = 16*FN consecutive weight rows over all of K.  Blocks
// are persistent: block b takes row blocks b, b + grid, ...  The bytes of
// each weight row are cut into chunks of CK bytes and wave w of the block
// takes chunks w, w + NW, ... of every row block, one after the other, so
// its copies run on across row-block boundaries.  One copy instruction
// moves 1 KB: 64 lanes x 16 consecutive bytes of 1024/CK rows, i.e. whole
// 128-byte lines.  A slot holds, for one chunk:
//   weights      [BN][CK] bytes (16-byte columns XOR-swizzled by row),
//   activations  [MX][XCK] bytes, the chunk's k range of MX token rows
//                (XCK = CK, or 2*CK for packed W4),
//   epilogue aux 64*IA dwords: sx of the MX tokens, sw of the BN columns
//                and bias pairs, gathered by 4-byte copies.
// The aux copy rides in every chunk so that the copy count per chunk, and
// with it every vmcnt wait, is a compile-time constant; at the end of a row
// block the wave's last slot holds what the epilogue needs.
//
// K tails: copies past the end of a row read clamped (valid) addresses,
// and the activation operand of every k past K is replaced by zero, so
// those products vanish.  Tokens past M read row M-1 and are never stored.
//
// At the end of a row block each wave adds its int32 partial fragments into
// an LDS buffer (exact, order-free), a barrier that waits on LDS only lets
// the copies stay in flight, and the fragments are finished by the waves in
// turn.  The buffer alternates between two halves by row-block parity, so
// a half is cleared by its reader one barrier before it is used again.
//
// A16 (fp16 activations, INT8 weights): the activation slot holds 2*CK
// bytes of each token row (CK k values), as for packed W4.  A lane's 16
// weight codes of a k-step (k = 16g .. 16g+15) are widened exactly to fp16
// and meet its two 16-byte activation columns in two
// v_mfma_f32_16x16x32_f16 (codes 0..7, then 8..15: the MFMA's k order is a
// summation order, the same for both operands).  fp32 partials are not
// order-free, so each wave writes its own partial fragments and the
// finishing wave adds them in wave order: the result does not depend on
// timing.

// Workgroup barrier over LDS traffic that leaves the global->LDS copies in
// flight: it waits for this wave's DS operations only (a release fence would
// also wait for the copies, which are LDS writes too), and keeps the
// compiler from moving memory accesses across it.  Correct only for LDS
// data that no copy in flight writes.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), no vmcnt wait
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// LDS stores issued while global->LDS copies are in flight.  Written as
// plain DS instructions because the compiler, unable to tell the
// destinations apart, would otherwise wait for every copy in flight before
// any LDS store.  The addresses never overlap a copy destination.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)ZQ_LPTR(p);
}
__device__ __forceinline__ void ds_add4(uint32_t addr, v4i v) {
  asm volatile(
      "ds_add_u32 %0, %1\n\t"
      "ds_add_u32 %0, %2 offset:4\n\t"
      "ds_add_u32 %0, %3 offset:8\n\t"
      "ds_add_u32 %0, %4 offset:12"
      :
      : "v"(addr), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3])
      : "memory");
}
__device__ __forceinline__ void ds_zero16(uint32_t addr) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v4i{0, 0, 0, 0})
               : "memory");
}
__device__ __forceinline__ void ds_write16(uint32_t addr, v4i v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Wait until at most `later` chunks of copies issued after the one needed
// are still in flight.
template <class C>
__device__ __forceinline__ void wait_chunks(int later) {
  if constexpr (C::D >= 4) {
    if (later >= 3) { wait_vmcnt<3 * C::P>(); return; }
  }
  if constexpr (C::D >= 3) {
    if (later >= 2) { wait_vmcnt<2 * C::P>(); return; }
  }
  if (later >= 1) { wait_vmcnt<C::P>(); return; }
  wait_vmcnt<0>();
}

// Cache policy of a global -> LDS copy: non-temporal (nt), for bytes read
// once per launch.
constexpr int kCopyNT = 2;

template <class C, bool CHK>
__device__ __forceinline__ void stream_issue(const GemmArgs &p, const char *W,
                                             const char *X, int ldw, int rb,
                                             int c, char *slot, int lane) {
  const int n0 = rb * C::BN;
  // every weight byte is copied once per launch: non-temporal for rings of
  // up to 16 token rows (3-5% faster per 16-token linear, same box A/B);
  // with 64 token rows it measured slower (NeoX attention output 20.5 ->
  // 22.0 us), so the larger rings keep the default policy
  constexpr int wpol = C::MX <= 16 ? kCopyNT : 0;
#pragma unroll
  for (int q = 0; q < C::IW; ++q) {
    const CopyAddr a = CHK ? stream_w_copy_chunked<C>(q, lane, rb, c, ldw)
                           : stream_w_copy<C>(q, lane, n0, c, p.N, ldw);
    __builtin_amdgcn_global_load_lds(ZQ_GPTR(W + a.goff), ZQ_LPTR(slot + a.lds),
                                     16, 0, wpol);
  }
  const int xrow = C::A16 ? 2 * p.K : p.K;     // activation row bytes
#pragma unroll
  for (int q = 0; q < C::IX; ++q) {
    const CopyAddr a = stream_x_copy<C>(q, lane, c, p.M, xrow);
    __builtin_amdgcn_global_load_lds(ZQ_GPTR(X + a.goff), ZQ_LPTR(slot + a.lds),
                                     16, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < C::IA; ++q) {
    const AuxElem a = stream_aux_elem<C>(q * 64 + lane, n0, p.M, p.N, p.G);
    const void *src = p.qw;                    // padding lanes: any dword
    if (a.src == kAuxSx) {
      if (p.sx) src = p.sx + a.index;
    } else if (a.src == kAuxSw) {
      if (p.sw) src = p.sw + a.index;
    } else if (a.src == kAuxBias) {
      if (p.bias) src = reinterpret_cast<const int *>(p.bias) + a.index;
    }
    __builtin_amdgcn_global_load_lds(ZQ_GPTR(src),
                                     ZQ_LPTR(slot + C::AOFF + q * 256), 4, 0,
                                     0);
  }
}

// slot: the ring slot of chunk c (weights); xs: the chunk's activation
// image (in the slot, or resident).
template <class C>
__device__ __forceinline__ void stream_compute(const GemmArgs &p,
                                               const char *slot,
                                               const char *xs, int c,
                                               int r16, int g,
                                               v4i (&acc)[C::FN][C::MF]) {
  const v4i zero = {0, 0, 0, 0};
  const int k0 = c * (C::W4 ? 2 * C::CK : C::CK);
#pragma unroll
  for (int s = 0; s < C::SPC; ++s) {
    v4i a[C::FN];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int row = fn * 16 + r16;
      a[fn] = ld16(slot + row * C::CK + (((4 * s + g) ^ (row & C::WSW)) << 4));
    }
    if constexpr (C::A16) {
      typedef float v4f __attribute__((ext_vector_type(4)));
      const bool kok = k0 + 64 * s + 16 * g < p.K;
      v4i wl[C::FN], wh[C::FN];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int w0 = a[fn][0], w1 = a[fn][1], w2 = a[fn][2], w3 = a[fn][3];
        wl[fn] = i8x8_to_f16x8(w0, w1);
        wh[fn] = i8x8_to_f16x8(w2, w3);
      }
#pragma unroll
      for (int fm = 0; fm < C::MF; ++fm) {
        int row = fm * 16 + r16;
        row = row < p.M ? row : p.M - 1;
        const char *xr = xs + row * C::XCK;
        const int cx = 8 * s + 2 * g;
        v4i b0 = ld16(xr + ((cx ^ (row & C::XSW)) << 4));
        v4i b1 = ld16(xr + (((cx + 1) ^ (row & C::XSW)) << 4));
        b0 = kok ? b0 : zero;
        b1 = kok ? b1 : zero;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          v4f f = __builtin_bit_cast(v4f, acc[fn][fm]);
          f = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(half8, wl[fn]), __builtin_bit_cast(half8, b0),
              f, 0, 0, 0);
          f = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(half8, wh[fn]), __builtin_bit_cast(half8, b1),
              f, 0, 0, 0);
          acc[fn][fm] = __builtin_bit_cast(v4i, f);
        }
      }
    } else if constexpr (!C::W4) {
      const bool kok = k0 + 64 * s + 16 * g < p.K;
#pragma unroll
      for (int fm = 0; fm < C::MF; ++fm) {
        int row = fm * 16 + r16;
        row = row < p.M ? row : p.M - 1;
        v4i b = ld16(xs + row * C::XCK +
                     (((4 * s + g) ^ (row & C::XSW)) << 4));
        b = kok ? b : zero;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fn][fm] = mfma_i8(a[fn], b, acc[fn][fm]);
      }
    } else {
      const bool kok = k0 + 128 * s + 32 * g < p.K;
#pragma unroll
      for (int fm = 0; fm < C::MF; ++fm) {
        int row = fm * 16 + r16;
        row = row < p.M ? row : p.M - 1;
        const char *xr = xs + row * C::XCK;
        const int cx = 8 * s + 2 * g;
        v4i b0 = ld16(xr + ((cx ^ (row & C::XSW)) << 4));
        v4i b1 = ld16(xr + (((cx + 1) ^ (row & C::XSW)) << 4));
        b0 = kok ? perm_even_odd(b0) : zero;
        b1 = kok ? perm_even_odd(b1) : zero;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          acc[fn][fm] = mfma_i8(unpack_w4(a[fn][0], a[fn][1]), b0, acc[fn][fm]);
          acc[fn][fm] = mfma_i8(unpack_w4(a[fn][2], a[fn][3]), b1, acc[fn][fm]);
        }
      }
    }
  }
}

// CHK: the weights are in the chunk-contiguous layout (stream_w_copy_chunked)
template <class C, bool RAW, bool CHK = false>
__global__ void __launch_bounds__(C::NT)
gemm_stream_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int ldw = C::W4 ? p.K / 2 : p.K;
  const char *W = static_cast<const char *>(p.qw);
  const char *X = reinterpret_cast<const char *>(p.qx);
  char *ring = lds + wave * (C::D * C::SLOT);
  char *xres = lds + C::NW * C::D * C::SLOT + wave * C::XRES;
  int *red = reinterpret_cast<int *>(lds + C::NW * (C::D * C::SLOT + C::XRES));

  const int NRB = (p.N + C::BN - 1) / C::BN;
  const int NC = (ldw + C::CK - 1) / C::CK;            // chunks per row
  const int ncw = NC > wave ? (NC - wave + C::NW - 1) / C::NW : 0;
  const int nact = NC < C::NW ? NC : C::NW;            // waves with chunks
  const int nrb = (NRB - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int total = ncw * nrb;

  for (int i = threadIdx.x; i < 2 * C::RED / 4; i += C::NT) red[i] = 0;
  lds_barrier();  // red[] cleared before any copy is issued

  if constexpr (C::XR > 0) {
    // this wave's activation chunks, once (the launcher guarantees
    // ncw <= XR); issued before the ring, so the first chunk wait covers
    // them, and read only by this wave
    const int xrow = p.K;
#pragma unroll
    for (int ic = 0; ic < C::XR; ++ic)
      if (ic < ncw) {
#pragma unroll
        for (int q = 0; q < C::IXC; ++q) {
          const CopyAddr a = stream_x_copy<C>(q, lane, wave + ic * C::NW, p.M, xrow);
          __builtin_amdgcn_global_load_lds(
              ZQ_GPTR(X + a.goff),
              ZQ_LPTR(xres + ic * C::XCH + (a.lds - C::XOFF)), 16, 0, 0);
        }
      }
  }

  // copy cursor: chunk j_issue = (row block index ir, chunk index ic)
  int j_issue = 0, ir = 0, ic = 0;
  auto issue_next = [&]() {
    stream_issue<C, CHK>(p, W, X, ldw, (int)blockIdx.x + ir * (int)gridDim.x,
                    wave + ic * C::NW,
                    ring + ((unsigned)j_issue % C::D) * C::SLOT, lane);
    ++j_issue;
    if (++ic == ncw) { ic = 0; ++ir; }
  };
#pragma unroll
  for (int d = 0; d < C::D - 1; ++d)
    if (j_issue < total) issue_next();

  int j = 0;
  for (int rbi = 0; rbi < nrb; ++rbi) {
    const int rb = (int)blockIdx.x + rbi * (int)gridDim.x;
    v4i acc[C::FN][C::MF];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < C::MF; ++fm) acc[fn][fm] = v4i{0, 0, 0, 0};

    for (int ci = 0; ci < ncw; ++ci, ++j) {
      if (j_issue < total) issue_next();
      wait_chunks<C>(j_issue - 1 - j);
      __builtin_amdgcn_sched_barrier(0);
      const char *slot = ring + ((unsigned)j % C::D) * C::SLOT;
      stream_compute<C>(p, slot,
                        C::XR > 0 ? xres + ci * C::XCH : slot + C::XOFF,
                        wave + ci * C::NW, r16, g, acc);
      __builtin_amdgcn_sched_barrier(0);
    }

    int *rh = red + (rbi & 1) * (C::RED / 4);
    constexpr int NPR = C::FN * C::MF;         // fragments per row block
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < C::MF; ++fm) {
        if constexpr (C::A16)
          ds_write16(lds_addr(&rh[((wave * NPR + fn * C::MF + fm) * kWave + lane) * 4]),
                     acc[fn][fm]);
        else
          ds_add4(lds_addr(&rh[((fn * C::MF + fm) * kWave + lane) * 4]),
                  acc[fn][fm]);
      }
    lds_barrier();

    if (wave < nact) {
      // the aux dwords of this row block sit in the slot of this wave's
      // last chunk of it
      const int *aux = reinterpret_cast<const int *>(
          ring + ((unsigned)(j - 1) % C::D) * C::SLOT + C::AOFF);
      for (int pr = wave; pr < C::FN * C::MF; pr += nact) {
        const int fn = pr / C::MF, fm = pr % C::MF;
        v4i a;
        if constexpr (C::A16) {
          // the waves' fp32 partials, added in wave order
          typedef float v4f __attribute__((ext_vector_type(4)));
          v4f sum = __builtin_bit_cast(
              v4f, *reinterpret_cast<const v4i *>(&rh[(pr * kWave + lane) * 4]));
#pragma unroll
          for (int w = 1; w < C::NW; ++w)
            sum += __builtin_bit_cast(
                v4f, *reinterpret_cast<const v4i *>(
                         &rh[((w * NPR + pr) * kWave + lane) * 4]));
          a = __builtin_bit_cast(v4i, sum);
        } else {
          int *rp = &rh[(pr * kWave + lane) * 4];
          a = *reinterpret_cast<const v4i *>(rp);
          ds_zero16(lds_addr(rp));
        }
        const int t = fm * 16 + r16;
        const int cb = fn * 16 + 4 * g;          // column within the row block
        const int nb = rb * C::BN + cb;
        QuadCol qc;
        float sxt = 0.0f;
        if constexpr (!RAW) {
          sxt = C::A16 ? 1.0f : __int_as_float(aux[t < p.M ? t : p.M - 1]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            qc.sw[r] = __int_as_float(aux[C::MX + cb + r]);
            const int bw = aux[C::MX + C::BN + (cb + r) / 2];
            const uint16_t hb = (uint16_t)(((cb + r) & 1) ? (bw >> 16) : bw);
            qc.b[r] = p.bias ? __builtin_bit_cast(half_t, hb) : (half_t)0.0f;
          }
        }
        store_quad<C::W4, RAW, C::A16>(p, t, nb, a, sxt, qc);
      }
    }
  }
}

// Number of compute units of the current device (cached per device; host
// threads may race to fill an entry, all with the same value).
static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess || v <= 0)
      v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <class C, bool RAW, bool CHK = false>
static hipError_t run_stream(const GemmArgs &a, hipStream_t s) {
  const int nrb = (a.N + C::BN - 1) / C::BN;
  const int cus = device_cus();
  const int grid = nrb < cus ? nrb : cus;
  hipLaunchKernelGGL((gemm_stream_kernel<C, RAW, CHK>), dim3(grid), dim3(C::NT),
                     0, s, a);
  return hipGetLastError();
}

// ==================================================================== gemv
// One token (M = 1): y[n] = dot(W[n, :], x).  MFMA would waste 15/16 of its
// work here, and the 16-row operand it needs makes every copy touch 16 rows
// at once; HBM delivers its full rate only when reads run through long
// contiguous windows.  So block b owns the rows [r0, r1), one contiguous
// byte range of W, cut into 1 KB pieces; wave w takes pieces w, w + NW, ...
// (the block's waves read one contiguous window), loads them into registers
// (16 bytes per lane, non-temporal: read once) with U pieces in flight, and
// multiplies them with v_dot4_i32_i8 against the matching activation bytes.
// The activation row (K bytes) is copied into LDS once at the start when it
// fits, else re-read from the caches.  A wave's
// sum for a row (DPP across the wave) is added into an LDS row sum; the
// epilogue runs once at the end of the block, with its scale and bias
// operands loaded before the weight stream.
//
// W4: the packed bytes are split as in the MFMA kernels into 16*q words
// (even k / odd k), the activation bytes permuted to match (once, when the
// row is staged in LDS; per piece when it is read from the caches), and the
// row sum shifted right by 4 at the end.  Rows must be a whole number of 1 KB pieces
// (K % 1024 == 0 for W8, K % 2048 == 0 for W4).
//
// XQ: the activation arrives as the fp16 row the previous linear wrote, and
// each block token-quantizes it while staging it into LDS: the block's
// maximum of |x| over the whole row (every block loads the whole row, so no
// other block's result is needed), S = amax / 127, and the codes from the
// same exact quantizer helper as the row-quantizer kernel, so codes, S and
// y equal those of the separate quantizer launch followed by this GEMM.
// Block 0 also writes the codes and S out.
template <int NW_, int U_, bool W4_, int XR_, bool A16_ = false,
          bool XQ_ = false>
struct Gemv {
  static constexpr int NW = NW_, U = U_;
  static constexpr bool W4 = W4_;
  // A16: fp16 activation row (2 bytes per k, held in LDS), INT8 weights;
  // fp32 row sums from v_dot2_f32_f16 on the widened codes
  static constexpr bool A16 = A16_;
  static constexpr bool XQ = XQ_;
  static constexpr int NT = NW * kWave;
  static constexpr int RMAX = 1024;   // rows per block
  // XR > 0: the activation row (at most XMAX bytes) is held in LDS, loaded
  // as XR 16-byte pieces per thread
  static constexpr int XR = XR_;
  static constexpr bool XL = XR > 0;
  static constexpr int XMAX = XR * NT * 16;
  static constexpr int L = XL ? 1 : (W4 ? 3 : 2);  // loads per piece
  static_assert(U * L < 64, "vmcnt range");
  static_assert(!A16 || (XL && !W4), "fp16 activations: W8, row in LDS");
  static_assert(!XQ || (XL && !A16), "quantized on load: codes in LDS");
};

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_i<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_i<0x141>(v);  // row_half_mirror
  v += dpp_i<0x140>(v);  // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ int dot16(v4i w, v4i x, int acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_sdot4(w[i], x[i], acc, false);
  return acc;
}

__device__ __forceinline__ void ds_add1(uint32_t addr, int v) {
  asm volatile("ds_add_u32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ void ds_add1f(uint32_t addr, float v) {
  asm volatile("ds_add_f32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// sum_i w_i * x_i over 8 fp16 pairs in fp32 (v_dot2_f32_f16); the vector
// elements are copied to scalars before the bit casts
__device__ __forceinline__ float fdot8(v4i w, v4i x, float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int wi = w[i], xi = x[i];
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, wi),
                                 __builtin_bit_cast(h2, xi), acc, false);
  }
  return acc;
}

template <class C, bool RAW>
__global__ void __launch_bounds__(C::NT)
gemm_gemv_kernel(GemmArgs p, int rpb, int interleave, int8_t *xq_codes,
                 float *xq_scale) {
  __shared__ int rowsum[C::RMAX];
  __shared__ __attribute__((aligned(1024))) char xs[C::XL ? C::XMAX : 16];
  __shared__ float xq_red[C::NW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ldw = C::W4 ? p.K / 2 : p.K;
  const int ppr = ldw >> 10;                   // pieces per row
  const int xbytes = C::A16 ? 2 * p.K : p.K;   // activation row bytes
  const int r0 = (int)blockIdx.x * rpb;
  const int r1 = r0 + rpb < p.N ? r0 + rpb : p.N;
  // piece order of a wave: interleaved (pieces wave, wave + NW, ... of the
  // block's range: one contiguous window per block) or by rows (all pieces
  // of rows wave, wave + NW, ...: one flush per row)
  int npieces;
  if (interleave) {
    const int tot = (r1 - r0) * ppr;
    npieces = tot > wave ? (tot - wave + C::NW - 1) / C::NW : 0;
  } else {
    const int nrw = r1 - r0 > wave ? (r1 - r0 - wave + C::NW - 1) / C::NW : 0;
    npieces = nrw * ppr;
  }
  const char *W = static_cast<const char *>(p.qw);
  const char *X = reinterpret_cast<const char *>(p.qx);

  // row sums cleared before any copy into LDS is issued
  for (int i = threadIdx.x; i < r1 - r0; i += C::NT) rowsum[i] = 0;

  // epilogue operands of the rows this thread finishes (i = tid + e*NT)
  // (kept as loaded bits, not converted, so that nothing waits for them
  // here; without a bias a valid dummy is read and ignored)
  constexpr int E = C::RMAX / C::NT;
  float esw[E];
  uint16_t ebits[E];
  float esx = 0.0f;
  if constexpr (!RAW) {
    esx = C::A16 || C::XQ ? 1.0f : p.sx[0];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int n = r0 + (int)threadIdx.x + e * C::NT;
      n = n < r1 ? n : r1 - 1;
      esw[e] = p.sw[n / p.G];
      ebits[e] = *(p.bias ? reinterpret_cast<const uint16_t *>(p.bias) + n
                          : reinterpret_cast<const uint16_t *>(p.sw));
    }
  }

  // activation row: loaded now (clamped, unconditional), stored into LDS
  // after the first weight loads are in flight.  Piece e of a thread holds
  // the 16 codes at k = off .. off + 15; XQ loads their 32 fp16 bytes.
  constexpr int XR = C::XL ? C::XR : 1;
  constexpr int XH = C::XQ ? 2 : 1;
  v4i xr[XR][XH];
  if constexpr (C::XL) {
#pragma unroll
    for (int e = 0; e < XR; ++e) {
      const int off = (e * C::NT + (int)threadIdx.x) * 16;
      if constexpr (C::XQ) {
        // only pieces inside the row (whole waves, K % 1024 == 0): the
        // 32-byte fp16 pieces past its end would be re-read by every block
        xr[e][0] = xr[e][1] = v4i{0, 0, 0, 0};
        if (off < p.K) {
          xr[e][0] = ld16(X + 2 * off);
          xr[e][1] = ld16(X + 2 * off + 16);
        }
      } else {
        xr[e][0] = ld16(X + (off < xbytes ? off : xbytes - 16));
      }
    }
  }

  v4i wv[C::U];
  v4i xv[C::U][C::XL ? 1 : (C::W4 ? 2 : 1)];
  // load cursor: piece wave + NW*li = row lr (relative to r0), piece lp of
  // that row; it stays on the last piece once there (extra loads re-read
  // it and are never used)
  // cursor step: sp pieces and sr rows, plus wr rows when the piece index
  // wraps past the row end
  const int sp = interleave ? C::NW - (C::NW / ppr) * ppr : 1;
  const int sr = interleave ? C::NW / ppr : 0;
  const int wr = interleave ? 1 : C::NW;
  const int lr0 = interleave ? wave / ppr : wave;
  const int lp0 = interleave ? wave - (wave / ppr) * ppr : 0;
  int li = 0, lr = lr0, lp = lp0;
  auto load = [&](int u) {
    const int kb = lp << 10;
    const int row = r0 + lr < r1 ? r0 + lr : r1 - 1;  // (a wave without pieces)
    const char *wp = W + (size_t)row * ldw + kb + lane * 16;
    wv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(wp));
    if constexpr (!C::XL) {
      if constexpr (C::W4) {
        xv[u][0] = ld16(X + 2 * (kb + lane * 16));
        xv[u][1] = ld16(X + 2 * (kb + lane * 16) + 16);
      } else {
        xv[u][0] = ld16(X + kb + lane * 16);
      }
    }
    {
      const bool adv = li < npieces - 1;
      int np = lp + sp, nr = lr + sr;
      const bool wrap = np >= ppr;
      np = wrap ? np - ppr : np;
      nr = wrap ? nr + wr : nr;
      lp = adv ? np : lp;
      lr = adv ? nr : lr;
    }
    ++li;
  };
#pragma unroll
  for (int u = 0; u < C::U; ++u) load(u);
  if constexpr (C::XQ) {
    // token-wise quantization of the row (K % 1024 == 0, so a wave's pieces
    // are all inside the row or all past its end)
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < XR; ++e) {
      const int off = (e * C::NT + (int)threadIdx.x) * 16;
      if (off < p.K) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const half8 x8 = __builtin_bit_cast(half8, xr[e][h]);
#pragma unroll
          for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)x8[i]));
        }
      }
    }
    m = wave_max(m);
    if (lane == 0) xq_red[wave] = m;
    lds_barrier();
    float amax = 0.0f;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) amax = fmaxf(amax, xq_red[w]);
    const Quantizer qz = make_quantizer(amax, 127.0f);
    esx = qz.s;
    const bool out = blockIdx.x == 0 && xq_codes != nullptr;
#pragma unroll
    for (int e = 0; e < XR; ++e) {
      const int off = (e * C::NT + (int)threadIdx.x) * 16;
      if (off < p.K) {
        float v[2][8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const half8 x8 = __builtin_bit_cast(half8, xr[e][h]);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[h][i] = (float)x8[i];
        }
        // amax is the max |x| of the row: the codes need no clamp
        const v2i lo = quant8_pack_rowmax(v[0], qz);
        const v2i hi = quant8_pack_rowmax(v[1], qz);
        const v4i c = {lo[0], lo[1], hi[0], hi[1]};
        *reinterpret_cast<v4i *>(xs + off) = C::W4 ? perm_even_odd(c) : c;
        if (out) *reinterpret_cast<v4i *>(xq_codes + off) = c;
      }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && xq_scale != nullptr)
      xq_scale[0] = qz.s;
  } else if constexpr (C::XL) {
#pragma unroll
    for (int e = 0; e < XR; ++e) {
      const int off = (e * C::NT + (int)threadIdx.x) * 16;
      if (off < xbytes)
        *reinterpret_cast<v4i *>(xs + off) =
            C::W4 ? perm_even_odd(xr[e][0]) : xr[e][0];
    }
  }
  lds_barrier();  // activation row and cleared row sums visible

  int acc = 0, ci = 0, cr = lr0, cp = lp0;
  float accf = 0.0f;
  for (int c0 = 0; c0 < npieces; c0 += C::U) {
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      if (c0 + u < npieces) {
        const int kb = cp << 10;
        if constexpr (C::A16) {
          // 16 codes (k = kb + 16 lane ..) against 16 fp16 activations
          const v4i x0 = ld16(xs + 2 * kb + lane * 32);
          const v4i x1 = ld16(xs + 2 * kb + lane * 32 + 16);
          accf = fdot8(i8x8_to_f16x8(wv[u][0], wv[u][1]), x0, accf);
          accf = fdot8(i8x8_to_f16x8(wv[u][2], wv[u][3]), x1, accf);
        } else if constexpr (C::W4) {
          v4i x0, x1;
          if constexpr (C::XL) {
            x0 = ld16(xs + 2 * kb + lane * 32);
            x1 = ld16(xs + 2 * kb + lane * 32 + 16);
          } else {
            x0 = xv[u][0];
            x1 = xv[u][1];
          }
          // (the row in LDS is stored in that order already)
          acc = dot16(unpack_w4(wv[u][0], wv[u][1]),
                      C::XL ? x0 : perm_even_odd(x0), acc);
          acc = dot16(unpack_w4(wv[u][2], wv[u][3]),
                      C::XL ? x1 : perm_even_odd(x1), acc);
        } else {
          const v4i x0 = C::XL ? ld16(xs + kb + lane * 16) : xv[u][0];
          acc = dot16(wv[u], x0, acc);
        }
        // next piece of this wave; flush the row sum when the row changes
        const int row = cr;
        cp += sp;
        cr += sr;
        const bool wrap = cp >= ppr;
        cp = wrap ? cp - ppr : cp;
        cr = wrap ? cr + wr : cr;
        if (cr != row || ci == npieces - 1) {
          if constexpr (C::A16) {
            const float sum = wave_sum(accf);
            if (lane == 0) ds_add1f(lds_addr(&rowsum[row]), sum);
            accf = 0.0f;
          } else {
            const int sum = wave_sum_i(acc);
            if (lane == 0) ds_add1(lds_addr(&rowsum[row]), C::W4 ? (sum >> 4) : sum);
            acc = 0;
          }
        }
        ++ci;
      }
      load(u);
    }
  }
  lds_barrier();  // row sums complete (the trailing re-reads stay in flight)

  // epilogue over the block's rows, consecutive threads on consecutive n
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = (int)threadIdx.x + e * C::NT;
    if (i < r1 - r0) {
      const int n = r0 + i;
      const int a = rowsum[i];
      if constexpr (RAW) {
        static_cast<int32_t *>(p.out)[n] = a;
      } else {
        const half_t b =
            p.bias ? __builtin_bit_cast(half_t, ebits[e]) : (half_t)0.0f;
        const float sc = esx * esw[e];
        const float af = C::A16 ? __builtin_bit_cast(float, a) : (float)a;
        static_cast<half_t *>(p.out)[n] =
            p.act == ZQ_ACT_GELU ? gelu_half(af, sc, b) : fma_half(af, sc, b);
      }
    }
  }
}

template <class C, bool RAW>
static hipError_t run_gemv(const GemmArgs &a, hipStream_t s, int bpc,
                           int interleave, int8_t *xq_codes = nullptr,
                           float *xq_scale = nullptr) {
  const int cus = device_cus();
  int grid = bpc * cus;
  if (grid > a.N) grid = a.N;
  int rpb = (a.N + grid - 1) / grid;
  if (rpb > C::RMAX) rpb = C::RMAX;
  grid = (a.N + rpb - 1) / rpb;
  hipLaunchKernelGGL((gemm_gemv_kernel<C, RAW>), dim3(grid), dim3(C::NT), 0,
                     s, a, rpb, interleave, xq_codes, xq_scale);
  return hipGetLastError();
}

// ========================================================= chunked layout
// Weights repacked for the rings of up to 16 token rows: [row block][chunk]
// [BN rows][CK bytes], so that every copy instruction of the ring reads
// 1 KB of consecutive bytes instead of 1024 / CK rows at a row stride (the
// row-major weights).  BN and CK are those of the 16-token ring for the
// shape, fixed here independently of the device (the rules of choose() /
// stream_resident at 256 compute units), so that a packed buffer stays
// valid everywhere.  2 to 16 tokens run that ring; one token runs
// gemm_chunk_gemv_kernel (the ring where its activation row would not fit).
//   W8: resident activations when K <= 6144 and N / 16 >= 512 (BN 16; CK 512
//       for K <= 4096, else 256); else BN 32 when 256 < N / 16 and
//       N / 32 <= 256, else BN 16; CK 256.
//   W4: BN 32; resident activations when K <= 6144 and N / 32 >= 512 (CK 256
//       packed bytes for K <= 4096, else 128); else CK 128.
// Returns false when the shape does not tile (N % BN, row bytes % CK).
bool chunked_layout(int N, int K, int bits, int *bn, int *ck, int *xr) {
  const bool w4 = bits == 4;
  const int ldw = w4 ? K / 2 : K;
  int b, c, x = 0;
  if (!w4) {
    if (K <= 6144 && N / 16 >= 512) {
      b = 16;
      x = K <= 4096 ? 2 : 6;
      c = K <= 4096 ? 512 : 256;
    } else {
      b = (N / 16 > 256 && N / 32 <= 256) ? 32 : 16;
      c = 256;
    }
  } else {
    b = 32;
    if (K <= 6144 && N / 32 >= 512) {
      x = K <= 4096 ? 2 : 6;
      c = K <= 4096 ? 256 : 128;
    } else {
      c = 128;
    }
  }
  if (bn) *bn = b;
  if (ck) *ck = c;
  if (xr) *xr = x;
  return N > 0 && K > 0 && N % b == 0 && ldw % c == 0;
}

// Row-major codes -> chunked layout, one thread per 16-byte unit of the
// output: unit u = ((rb * NC + c) * BN + r) * (CK / 16) + j holds bytes
// c * CK + 16 j .. + 15 of row rb * BN + r.
__global__ void __launch_bounds__(256)
chunk_pack_kernel(const char *__restrict__ qw, int ldw, int bn, int ck,
                  size_t units, char *__restrict__ out) {
  const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int jn = ck / 16;
  const int j = (int)(u % jn);
  const size_t rc = u / jn;  // (rb * NC + c) * BN + r
  const int r = (int)(rc % bn);
  const size_t chunk = rc / bn;
  const int nc = ldw / ck;
  const size_t rb = chunk / nc;
  const int c = (int)(chunk % nc);
  const size_t src = (rb * bn + r) * (size_t)ldw + (size_t)c * ck + 16 * j;
  *reinterpret_cast<v4i *>(out + u * 16) =
      *reinterpret_cast<const v4i *>(qw + src);
}

hipError_t launch_pack_chunked(const void *qw, int N, int K, int bits,
                               void *out, hipStream_t s) {
  int bn, ck;
  chunked_layout(N, K, bits, &bn, &ck, nullptr);
  const int ldw = bits == 4 ? K / 2 : K;
  const size_t units = (size_t)N * ldw / 16;
  const size_t grid = (units + 255) / 256;
  hipLaunchKernelGGL(chunk_pack_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const char *>(qw), ldw, bn, ck, units,
                     static_cast<char *>(out));
  return hipGetLastError();
}

template <bool W4, bool RAW>
static hipError_t run_chunked(const GemmArgs &a, hipStream_t s) {
  int bn, ck, xr;
  chunked_layout(a.N, a.K, a.bits, &bn, &ck, &xr);
  if constexpr (W4) {
    if (xr == 2)
      return run_stream<Stream<2, 16, 4, 256, 2, true, false, 2>, RAW, true>(a, s);
    if (xr == 6)
      return run_stream<Stream<2, 16, 4, 128, 3, true, false, 6>, RAW, true>(a, s);
    return run_stream<Stream<2, 16, 4, 128, 4, true>, RAW, true>(a, s);
  } else {
    if (xr == 2)
      return run_stream<Stream<1, 16, 4, 512, 2, false, false, 2>, RAW, true>(a, s);
    if (xr == 6)
      return run_stream<Stream<1, 16, 4, 256, 3, false, false, 6>, RAW, true>(a, s);
    if (bn == 32)
      return run_stream<Stream<2, 16, 4, 256, 3, false>, RAW, true>(a, s);
    return run_stream<Stream<1, 16, 4, 256, 4, false>, RAW, true>(a, s);
  }
}

// One token over the chunked layout.  A row block (BN rows, all K) is one
// contiguous range of BN * R bytes (R = row bytes), cut into 1 KB pieces of
// 1024 / CK rows x CK bytes.  Workgroup b owns rbpb consecutive row blocks
// (one, as launched); wave w of its NW waves reads pieces w, w + NW, ... of
// that range (one contiguous window per workgroup), 16 bytes per lane, U
// pieces in flight (non-temporal: read once).  The pieces per chunk (PPC)
// are a multiple of NW, so a wave meets the same piece positions in every
// chunk and each lane always sees the same weight rows (RS = PPC / NW of
// them, one accumulator each).  The lanes of a row (CK / 16 consecutive
// lanes) add their partial dot products with DPP at the end of the row
// block; the epilogue runs once per workgroup, with its operands loaded
// before the weight stream.  The activation row is staged in LDS once (W4:
// each 16-byte group in the unpacked nibble order).
template <int BN_, int CK_, int NW_, bool W4_>
struct ChunkGemv {
  static constexpr int BN = BN_, CK = CK_, NW = NW_, U = 8;
  static constexpr bool W4 = W4_;
  static constexpr int NT = NW * kWave;
  static constexpr int PPC = BN * CK / 1024;  // pieces per chunk
  static constexpr int RPP = 1024 / CK;       // rows per piece
  static constexpr int LPR = CK / 16;         // lanes per row
  // NW <= PPC: each wave owns RS = PPC / NW piece positions of every chunk;
  // NW > PPC: WPP = NW / PPC waves share a position, each taking every WPP-th
  // chunk, and their row sums meet in LDS by atomic adds
  static constexpr int RS = NW <= PPC ? PPC / NW : 1;
  static constexpr int WPP = NW <= PPC ? 1 : NW / PPC;
  static constexpr int RMAX = 1024;           // rows per block
  static constexpr int XMAX = 32768;          // activation bytes in LDS
  static constexpr int XR = XMAX / (NT * 16);
  // every piece position of a chunk belongs to exactly one wave, so each
  // row's sum is written by one wave
  static_assert(PPC % NW == 0 || NW % PPC == 0, "pieces per chunk vs waves");
  static_assert(U % RS == 0, "accumulator of a piece known at compile time");
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row lanes");
};

template <class C>
__device__ __forceinline__ int row_lanes_sum(int v) {
  v += dpp_i<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_i<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_i<0x141>(v);   // row_half_mirror: 8-lane sums
  if constexpr (C::LPR >= 16) v += dpp_i<0x140>(v);  // row_mirror: 16 lanes
  if constexpr (C::LPR == 32) v += __shfl_xor(v, 16);
  return v;
}

template <class C, bool RAW>
__global__ void __launch_bounds__(C::NT)
gemm_chunk_gemv_kernel(GemmArgs p, int rbpb) {
  __shared__ int rowsum[C::RMAX];
  __shared__ __attribute__((aligned(1024))) char xs[C::XMAX];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ldw = C::W4 ? p.K / 2 : p.K;
  const int NC = ldw / C::CK;                 // chunks per row block
  const int NRB = p.N / C::BN;
  const int rb0 = (int)blockIdx.x * rbpb;
  const int rb1 = rb0 + rbpb < NRB ? rb0 + rbpb : NRB;
  const int nrows = (rb1 - rb0) * C::BN;
  const int per_rb = NC * C::PPC;             // pieces per row block
  const int tot = (rb1 - rb0) * per_rb;       // pieces of the block
  // pieces of this wave: wave, wave + NW, ... (per_rb % NW == 0)
  const int npieces = tot > wave ? (tot - wave + C::NW - 1) / C::NW : 0;
  const char *W = static_cast<const char *>(p.qw) +
                  (size_t)rb0 * per_rb * 1024 + lane * 16;
  const char *X = reinterpret_cast<const char *>(p.qx);
  if constexpr (C::WPP > 1) {
    // shared positions add their partial row sums: start from zero
    for (int i = threadIdx.x; i < nrows; i += C::NT) rowsum[i] = 0;
  }

  // epilogue operands of the rows this thread finishes (i = tid + e*NT)
  constexpr int E = C::RMAX / C::NT;
  float esw[E];
  uint16_t ebits[E];
  float esx = 0.0f;
  if constexpr (!RAW) {
    esx = p.sx[0];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int n = rb0 * C::BN + (int)threadIdx.x + e * C::NT;
      n = n < rb1 * C::BN ? n : rb1 * C::BN - 1;
      esw[e] = p.sw[n / p.G];
      ebits[e] = *(p.bias ? reinterpret_cast<const uint16_t *>(p.bias) + n
                          : reinterpret_cast<const uint16_t *>(p.sw));
    }
  }
  // the activation row (K bytes), loaded now, stored after the first
  // weight loads are in flight
  v4i xr[C::XR];
#pragma unroll
  for (int e = 0; e < C::XR; ++e) {
    const int off = (e * C::NT + (int)threadIdx.x) * 16;
    xr[e] = ld16(X + (off < p.K ? off : p.K - 16));
  }

  // load cursor: piece g = wave + NW * li of the block's range, its chunk c
  // within the row block (clamped to the last piece once there)
  const int q0 = wave < tot ? wave : tot - 1;
  int li = 0, lq = q0;
  v4i wv[C::U];
  auto load = [&](int u) {
    wv[u] = __builtin_nontemporal_load(
        reinterpret_cast<const v4i *>(W + (size_t)lq * 1024));
    lq = li < npieces - 1 ? lq + C::NW : lq;
    ++li;
  };
#pragma unroll
  for (int u = 0; u < C::U; ++u) load(u);
#pragma unroll
  for (int e = 0; e < C::XR; ++e) {
    const int off = (e * C::NT + (int)threadIdx.x) * 16;
    if (off < p.K)
      *reinterpret_cast<v4i *>(xs + off) = C::W4 ? perm_even_odd(xr[e]) : xr[e];
  }
  lds_barrier();  // activation row visible

  // this lane's rows (within a row block) and 16-byte column of a chunk
  const int p0 = wave % C::PPC;
  const int jcol = lane % C::LPR;
  int acc[C::RS];
#pragma unroll
  for (int i = 0; i < C::RS; ++i) acc[i] = 0;
  // consume cursor: piece index within the row block (wi) and row block
  int ci = 0, wi = q0 % per_rb, rbl = q0 / per_rb;
  for (int c0 = 0; c0 < npieces; c0 += C::U) {
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      if (c0 + u < npieces) {
        const int i = u % C::RS;  // (unrolled: a constant)
        const int c = wi / C::PPC;                       // chunk
        const int kb = c * C::CK + 16 * jcol;            // weight byte in row
        if constexpr (C::W4) {
          const v4i x0 = ld16(xs + 2 * kb);
          const v4i x1 = ld16(xs + 2 * kb + 16);
          acc[i] = dot16(unpack_w4(wv[u][0], wv[u][1]), x0, acc[i]);
          acc[i] = dot16(unpack_w4(wv[u][2], wv[u][3]), x1, acc[i]);
        } else {
          acc[i] = dot16(wv[u], ld16(xs + kb), acc[i]);
        }
        int nw = wi + C::NW;
        const bool wrap = nw >= per_rb;
        if (wrap || ci == npieces - 1) {
          // end of this wave's share of the row block: row sums
#pragma unroll
          for (int r = 0; r < C::RS; ++r) {
            const int sum = row_lanes_sum<C>(acc[r]);
            if (jcol == 0) {
              const int row = (p0 + C::NW * r) * C::RPP + lane / C::LPR;
              const int v = C::W4 ? (sum >> 4) : sum;
              if constexpr (C::WPP > 1)
                ds_add1(lds_addr(&rowsum[rbl * C::BN + row]), v);
              else
                rowsum[rbl * C::BN + row] = v;
            }
            acc[r] = 0;
          }
        }
        wi = wrap ? nw - per_rb : nw;
        rbl = wrap ? rbl + 1 : rbl;
        ++ci;
      }
      load(u);
    }
  }
  lds_barrier();  // row sums complete (the trailing re-reads stay in flight)

#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = (int)threadIdx.x + e * C::NT;
    if (i < nrows) {
      const int n = rb0 * C::BN + i;
      const int a = rowsum[i];
      if constexpr (RAW) {
        static_cast<int32_t *>(p.out)[n] = a;
      } else {
        const half_t b =
            p.bias ? __builtin_bit_cast(half_t, ebits[e]) : (half_t)0.0f;
        const float sc = esx * esw[e];
        static_cast<half_t *>(p.out)[n] =
            p.act == ZQ_ACT_GELU ? gelu_half((float)a, sc, b)
                                 : fma_half((float)a, sc, b);
      }
    }
  }
}

template <class C, bool RAW>
static hipError_t run_chunk_gemv(const GemmArgs &a, hipStream_t s) {
  // one row block per workgroup (against up to two workgroups per CU with
  // several row blocks each: the eight GPT-J / NeoX one-token linears 114.3
  // -> 112.4 us; 16 pieces in flight instead of 8: 123.1 / 126.5 us)
  const int nrb = a.N / C::BN;
  hipLaunchKernelGGL((gemm_chunk_gemv_kernel<C, RAW>), dim3(nrb), dim3(C::NT),
                     0, s, a, 1);
  return hipGetLastError();
}

// the one-token kernel over the chunked layout applies while the activation
// row fits its LDS image
static bool chunk_gemv_ok(int M, int K) { return M == 1 && K <= 32768; }

// Waves per workgroup of the one-token kernel: 8 (more bytes in flight per
// workgroup) where the row blocks number fewer than the CUs, or fewer than
// two per CU and hold at most 64 KB each; else 4.  Measured, 4 -> 8 waves
// (us): NeoX FFN2 19.5 -> 16.9, attention output 9.8 -> 9.5, GPT-J
// attention output 5.88 -> 5.51, but GPT-J FFN2 (256 KB row blocks)
// 13.9 -> 15.8.  ZQ_CGEMV_NW=<4|8> forces one where it applies (tuning aid).
static int chunk_gemv_waves(int N, int K, int bits) {
  int bn, ck;
  chunked_layout(N, K, bits, &bn, &ck, nullptr);
  const int nc = (bits == 4 ? K / 2 : K) / ck;
  const int ppc = bn * ck / 1024;
  const bool ok8 = ppc == 8 || nc % 2 == 0;  // per-row-block pieces % 8
  static const int forced = [] {
    const char *e = getenv("ZQ_CGEMV_NW");
    return e ? atoi(e) : 0;
  }();
  if (forced == 4) return 4;
  if (forced == 8) return ok8 ? 8 : 4;
  const int nrb = N / bn, cus = device_cus();
  const long rb_bytes = (long)bn * (bits == 4 ? K / 2 : K);
  return ok8 && (nrb < cus || (nrb < 2 * cus && rb_bytes <= 65536)) ? 8 : 4;
}

template <int NW, bool W4, bool RAW>
static hipError_t run_chunked_gemv_nw(const GemmArgs &a, int bn, int ck,
                                      hipStream_t s) {
  if constexpr (W4) {
    if (ck == 256) return run_chunk_gemv<ChunkGemv<32, 256, NW, true>, RAW>(a, s);
    return run_chunk_gemv<ChunkGemv<32, 128, NW, true>, RAW>(a, s);
  } else {
    if (ck == 512) return run_chunk_gemv<ChunkGemv<16, 512, NW, false>, RAW>(a, s);
    if (bn == 32) return run_chunk_gemv<ChunkGemv<32, 256, NW, false>, RAW>(a, s);
    return run_chunk_gemv<ChunkGemv<16, 256, NW, false>, RAW>(a, s);
  }
}

template <bool W4, bool RAW>
static hipError_t run_chunked_gemv(const GemmArgs &a, hipStream_t s) {
  int bn, ck;
  chunked_layout(a.N, a.K, a.bits, &bn, &ck, nullptr);
  if (chunk_gemv_waves(a.N, a.K, a.bits) == 8)
    return run_chunked_gemv_nw<8, W4, RAW>(a, bn, ck, s);
  return run_chunked_gemv_nw<4, W4, RAW>(a, bn, ck, s);
}

hipError_t launch_gemm_chunked(const GemmArgs &a, hipStream_t s) {
  if (chunk_gemv_ok(a.M, a.K)) {
    if (a.bits == 4)
      return a.raw_i32 ? run_chunked_gemv<true, true>(a, s)
                       : run_chunked_gemv<true, false>(a, s);
    return a.raw_i32 ? run_chunked_gemv<false, true>(a, s)
                     : run_chunked_gemv<false, false>(a, s);
  }
  if (a.bits == 4)
    return a.raw_i32 ? run_chunked<true, true>(a, s)
                     : run_chunked<true, false>(a, s);
  return a.raw_i32 ? run_chunked<false, true>(a, s)
                   : run_chunked<false, false>(a, s);
}

int describe_gemm_chunked_plan(int M, int N, int K, int bits, char *buf,
                               int len) {
  int bn, ck, xr;
  chunked_layout(N, K, bits, &bn, &ck, &xr);
  const int nrb = N / bn;
  if (chunk_gemv_ok(M, K))
    return snprintf(buf, len,
                    "chunked gemv BN=%d CK=%d NW=%d U=8 W%d row_blocks=%d "
                    "grid=%d", bn, ck, chunk_gemv_waves(N, K, bits), bits,
                    nrb, nrb);
  return snprintf(buf, len,
                  "chunked stream BN=%d CK=%d MX=16 NW=4 W%d%s M=%d "
                  "row_blocks=%d grid=%d",
                  bn, ck, bits, xr ? (xr == 2 ? " xres=2" : " xres=6") : "", M,
                  nrb, nrb < device_cus() ? nrb : device_cus());
}

// ================================================================ dispatch
template <class C, bool RAW>
static hipError_t run_tiled(const GemmArgs &a, hipStream_t s) {
  const int tiles = ((a.N + C::BN - 1) / C::BN) * ((a.M + C::BM - 1) / C::BM);
  hipLaunchKernelGGL((gemm_tiled_kernel<C, RAW>), dim3(tiles), dim3(C::NT), 0,
                     s, a);
  return hipGetLastError();
}

// The ping-pong kernel takes whole tiles: N a multiple of BN, K a multiple
// of the stage width with at least S stages, and (fused epilogue) group
// scales constant over each 32-column fragment and a 4-byte-aligned bias
// (both gathered as words).  Other problems run the same tile shape in
// gemm_tiled_kernel; the results are the same either way.
template <class C, bool RAW>
static hipError_t run_pingpong(const GemmArgs &a, hipStream_t s) {
  const bool fits = a.N % C::BN == 0 && a.K % C::KPS == 0 &&
                    a.K / C::KPS >= C::S &&
                    (RAW || (a.G % 32 == 0 &&
                             (!a.bias || ((uintptr_t)a.bias & 3) == 0)));
  if (!fits) return run_tiled<C, RAW>(a, s);
  const int tiles_m = (a.M + C::BM - 1) / C::BM, tiles_n = a.N / C::BN;
  const int nt = tiles_m * tiles_n;
  const int grid = nt < device_cus() ? nt : device_cus();
  hipLaunchKernelGGL((gemm_pingpong_kernel<C, RAW>), dim3(grid), dim3(C::NT),
                     0, s, a, tiles_m, tiles_n);
  return hipGetLastError();
}

template <class C, bool RAW>
static hipError_t run_skinny(const GemmArgs &a, hipStream_t s) {
  const int blocks = (a.N + C::BN - 1) / C::BN;
  hipLaunchKernelGGL((gemm_skinny_kernel<C, RAW>), dim3(blocks), dim3(C::NT),
                     0, s, a);
  return hipGetLastError();
}

// Tiled configurations: {BN, BM, WN, WM, stages, stage k-bytes}.
struct TileCfg {
  int bn, bm, wn, wm, s, kb;
  int persist;  // 1: gemm_pingpong_kernel (whole tiles only, else
                // gemm_tiled_kernel with the same tile; see run_pingpong)
};
static const TileCfg kTileCfgs[] = {
    {128, 128, 64, 64, 2, 128},    // 0: 4 waves
    {256, 128, 128, 64, 2, 128},   // 1: 4 waves
    {128, 256, 64, 128, 2, 128},   // 2: 4 waves
    {256, 256, 128, 128, 2, 128},  // 3: 4 waves
    {128, 128, 64, 64, 3, 128},    // 4: 4 waves
    {256, 256, 128, 64, 2, 128},   // 5: 8 waves
    {256, 128, 128, 64, 3, 128},   // 6: 4 waves
    {192, 256, 96, 128, 2, 128},   // 7: 4 waves
    {192, 128, 96, 64, 2, 128},    // 8: 4 waves
    {128, 192, 64, 96, 2, 128},    // 9: 4 waves
    {256, 128, 64, 64, 3, 128},    // 10: 8 waves
    {128, 256, 64, 64, 3, 128},    // 11: 8 waves
    {256, 256, 64, 64, 2, 128},    // 12: 16 waves
    {192, 256, 64, 64, 2, 128},    // 13: 12 waves
    {288, 128, 96, 32, 2, 128},    // 14: 12 waves
    {96, 128, 96, 32, 3, 128},     // 15: 4 waves
    {256, 256, 64, 64, 4, 64},   // 16: 16 waves, W8 only
    {256, 256, 128, 64, 4, 64},  // 17: 8 waves, W8 only
    {192, 256, 64, 64, 4, 64},   // 18: 12 waves, W8 only
    {128, 256, 64, 64, 5, 64},   // 19: 8 waves, W8 only
    {128, 128, 64, 64, 6, 64},   // 20: 4 waves, W8 only
    {128, 64, 64, 32, 6, 128},   // 21: 4 waves (decode-sized M)
    {64, 64, 32, 32, 8, 128},    // 22: 4 waves
    {64, 64, 32, 32, 12, 64},    // 23: 4 waves, W8 only
    {128, 32, 64, 32, 6, 128},   // 24: 2 waves
    {64, 64, 32, 32, 9, 128},    // 25: 4 waves
    {64, 32, 32, 32, 10, 128},   // 26: 2 waves
    {64, 64, 64, 32, 8, 128},    // 27: 2 waves
    // persistent ping-pong (two wave groups alternating memory and
    // compute), 8 waves of 64 outputs x 128 tokens, 3-stage ring: W4 only
    {256, 256, 64, 128, 3, 128, 1},  // 28
};
constexpr int kNumTileCfgs = sizeof(kTileCfgs) / sizeof(kTileCfgs[0]);

template <bool W4, bool RAW>
static hipError_t run_tile_cfg(int id, const GemmArgs &a, hipStream_t s) {
  switch (id) {
    case 0: return run_tiled<Tile<128, 128, 64, 64, 2, W4>, RAW>(a, s);
    case 1: return run_tiled<Tile<256, 128, 128, 64, 2, W4>, RAW>(a, s);
    case 2: return run_tiled<Tile<128, 256, 64, 128, 2, W4>, RAW>(a, s);
    case 3: return run_tiled<Tile<256, 256, 128, 128, 2, W4>, RAW>(a, s);
    case 4: return run_tiled<Tile<128, 128, 64, 64, 3, W4>, RAW>(a, s);
    case 5: return run_tiled<Tile<256, 256, 128, 64, 2, W4>, RAW>(a, s);
    case 6: return run_tiled<Tile<256, 128, 128, 64, 3, W4>, RAW>(a, s);
    case 7: return run_tiled<Tile<192, 256, 96, 128, 2, W4>, RAW>(a, s);
    case 8: return run_tiled<Tile<192, 128, 96, 64, 2, W4>, RAW>(a, s);
    case 9: return run_tiled<Tile<128, 192, 64, 96, 2, W4>, RAW>(a, s);
    case 10: return run_tiled<Tile<256, 128, 64, 64, 3, W4>, RAW>(a, s);
    case 11: return run_tiled<Tile<128, 256, 64, 64, 3, W4>, RAW>(a, s);
    case 13: return run_tiled<Tile<192, 256, 64, 64, 2, W4>, RAW>(a, s);
    case 14: return run_tiled<Tile<288, 128, 96, 32, 2, W4>, RAW>(a, s);
    case 15: return run_tiled<Tile<96, 128, 96, 32, 3, W4>, RAW>(a, s);
    case 16: if constexpr (!W4) return run_tiled<Tile<256, 256, 64, 64, 4, W4, 64>, RAW>(a, s); break;
    case 17: if constexpr (!W4) return run_tiled<Tile<256, 256, 128, 64, 4, W4, 64>, RAW>(a, s); break;
    case 18: if constexpr (!W4) return run_tiled<Tile<192, 256, 64, 64, 4, W4, 64>, RAW>(a, s); break;
    case 19: if constexpr (!W4) return run_tiled<Tile<128, 256, 64, 64, 5, W4, 64>, RAW>(a, s); break;
    case 20: if constexpr (!W4) return run_tiled<Tile<128, 128, 64, 64, 6, W4, 64>, RAW>(a, s); break;
    case 21: return run_tiled<Tile<128, 64, 64, 32, 6, W4>, RAW>(a, s);
    case 22: return run_tiled<Tile<64, 64, 32, 32, 8, W4>, RAW>(a, s);
    case 23: if constexpr (!W4) return run_tiled<Tile<64, 64, 32, 32, 12, W4, 64>, RAW>(a, s); break;
    case 24: return run_tiled<Tile<128, 32, 64, 32, 6, W4>, RAW>(a, s);
    case 25: return run_tiled<Tile<64, 64, 32, 32, 9, W4>, RAW>(a, s);
    case 26: return run_tiled<Tile<64, 32, 32, 32, 10, W4>, RAW>(a, s);
    case 27: return run_tiled<Tile<64, 64, 64, 32, 8, W4>, RAW>(a, s);
    case 28: if constexpr (W4) return run_pingpong<Tile<256, 256, 64, 128, 3, W4>, RAW>(a, s); break;
  }
  return run_tiled<Tile<256, 256, 64, 64, 2, W4>, RAW>(a, s);
}

enum PlanKind { kSkinny = 0, kTiled = 1, kStream = 2, kGemv = 3 };
struct Plan {
  PlanKind kind;
  int mf;   // skinny: 16-token fragments
  int cfg;  // tiled: index into kTileCfgs
  bool tuned = false;  // taken from the schedule table
};

// W8 rings of 16 token rows: 32-row weight blocks when 16-row blocks would
// outnumber the compute units and 32-row blocks would not.
static bool stream_w8_wide(int N) {
  const int cus = device_cus();
  return (N + 15) / 16 > cus && (N + 31) / 32 <= cus;
}

// Token rows a streaming ring holds: 1, 16, 32 or 64.
static int stream_mx(int M) {
  return M == 1 ? 1 : M <= 16 ? 16 : M <= 32 ? 32 : 64;
}

static int forced_xres() {
  static int v = [] {
    const char *e = getenv("ZQ_XRES");
    return e ? atoi(e) : -1;
  }();
  return v;
}

// Rings of 2 .. 16 token rows with resident activations (XR > 0): chosen
// when every workgroup takes at least two row blocks (the activations are
// then copied once instead of once per row block) and a wave's chunks fit
// the resident region (four waves; row blocks of 16 rows for W8, 32 for
// W4).  Returns XR, or 0 for the plain ring:
//   2: K <= 4096, chunks of 512 weight bytes (W4: 256), two ring slots;
//   6: K <= 6144, chunks of 256 weight bytes (W4: 128), three ring slots.
// Longer chunks make each copy instruction read longer runs of a weight row
// (GPT-J-6B FFN1, 16 x 16384 x 4096: 16.7 -> 15.9 us); the deeper ring of
// the 256-byte chunks gained nothing (5 slots against 3: 13.2 / 13.1 us
// for 16 x 12288 x 4096).  (ZQ_XRES=0 turns it off, 1 forces it wherever a
// wave's chunks fit: tuning aids.)
static int stream_resident(int M, int N, int K, int bits) {
  if (M < 2 || M > 16 || (N & 1) || forced_xres() == 0 || K > 6144) return 0;
  const int bn = bits == 4 ? 32 : 16;
  const int nrb = (N + bn - 1) / bn;
  if (forced_xres() < 1 && nrb < 2 * device_cus()) return 0;
  return K <= 4096 ? 2 : 6;
}

static bool w8_only(int cfg) {
  return (cfg >= 16 && cfg <= 20) || cfg == 23;
}
static bool w4_only(int cfg) { return cfg == 28; }

// Whether a plan of this kind / tile applies to a problem.  The tiled
// kernels take any M and N; the decode kernels have their own limits.
static bool plan_applies(PlanKind kind, int cfg, int M, int N, int K, int bits) {
  const int ldw = bits == 4 ? K / 2 : K;
  switch (kind) {
    case kGemv: return M == 1 && ldw % 1024 == 0;
    case kStream: return M >= 1 && M <= 64 && (N & 1) == 0;
    case kSkinny: return M >= 1 && M <= 64;
    case kTiled:
      return cfg >= 0 && cfg < kNumTileCfgs && !(bits == 4 && w8_only(cfg)) &&
             !(bits == 8 && w4_only(cfg));
  }
  return false;
}

// The decode kernels' launch parameters follow from M.
static Plan make_plan(PlanKind kind, int cfg, int M, bool tuned) {
  Plan p{kind, 0, cfg, tuned};
  if (kind == kSkinny) p.mf = (M + 15) / 16;
  if (kind == kStream) p.mf = stream_mx(M);
  if (kind == kGemv) p.mf = 1;
  if (kind != kTiled) p.cfg = 0;
  return p;
}

// ------------------------------------------------------- schedule table
// The pages profile several schedules per input-size combination and keep
// the best one per batch x seqlen.  Here a process-wide table maps
// (bits, N, K, M range) to a plan; the tuner fills it by timing every plan
// that applies, and choose() looks it up before its own rules.  The
// generation counter changes with every edit, so captured launch sequences
// know when their plans went stale.
struct SchedEntry {
  int bits, N, K, mlo, mhi;
  PlanKind kind;
  int cfg;
};
static std::mutex g_sched_mu;
static std::vector<SchedEntry> g_sched;
static std::atomic<unsigned> g_sched_gen{0};

static bool sched_lookup(int M, int N, int K, int bits, Plan *out) {
  std::lock_guard<std::mutex> lk(g_sched_mu);
  for (const SchedEntry &e : g_sched)
    if (e.bits == bits && e.N == N && e.K == K && M >= e.mlo && M <= e.mhi) {
      *out = make_plan(e.kind, e.cfg, M, true);
      return true;
    }
  return false;
}

// Replaces what the table holds for the same (bits, N, K) over [mlo, mhi]
// (overlapping entries are trimmed or split).
static void sched_put_locked(const SchedEntry &n) {
  std::vector<SchedEntry> keep;
  for (const SchedEntry &e : g_sched) {
    if (e.bits != n.bits || e.N != n.N || e.K != n.K || e.mhi < n.mlo ||
        e.mlo > n.mhi) {
      keep.push_back(e);
      continue;
    }
    if (e.mlo < n.mlo) {
      SchedEntry l = e;
      l.mhi = n.mlo - 1;
      keep.push_back(l);
    }
    if (e.mhi > n.mhi) {
      SchedEntry r = e;
      r.mlo = n.mhi + 1;
      keep.push_back(r);
    }
  }
  keep.push_back(n);
  g_sched.swap(keep);
}

// ZQ_GEMM_TILE=<index> forces one tiled configuration (tuning aid).
static int forced_tile() {
  static int v = [] {
    const char *e = getenv("ZQ_GEMM_TILE");
    if (!e) return -1;
    const int i = atoi(e);
    return (i >= 0 && i < kNumTileCfgs) ? i : -1;
  }();
  return v;
}

// Schedule selection by problem shape (the pages pick, per batch x seqlen,
// the tiling with the least waste).  Decode-sized M (<= 64) goes to the
// weight-streaming kernels, or for 17 .. 64 tokens over wide N to 64x64
// tiles with a deep copy ring.  Otherwise, from measured sweeps of every
// configuration (the schedule tuner over the five workloads' shapes at 128
// to 16384 tokens):
//  * when one round of tiles covers the problem: the smallest of 64x64,
//    128x64, 96x128 and 128x128 (deep-ring tiles, one block per CU) whose
//    tile count fits the compute units.  Every tile runs the whole K loop
//    and its per-stage MFMA work shrinks with the tile, so with a single
//    round the smallest tile that still fits finishes first (up to 1.7x
//    over 96x128 when K is long);
//  * W4 with K < 4096: 128x128 with two stages (two blocks per CU, so one
//    block's prologue and epilogue overlap the other's main loop);
//  * otherwise the candidate with the best score = fill x quality, where
//    fill is the fraction of the CU slots that the rounds of tiles keep busy
//    (tiles / (rounds x slots)) and quality the measured per-CU efficiency
//    of the configuration relative to 256x256 with 16 waves.
struct Candidate {
  int cfg, slots_per_cu;
  double quality;
};
static const Candidate kW8Candidates[] = {
    {12, 1, 1.00},  // 256x256, 16 waves
    {13, 1, 0.95},  // 192x256, 12 waves
    {14, 1, 0.85},  // 288x128, 12 waves
    {0, 2, 0.87},   // 128x128, 4 waves, two blocks per CU
};

// One-round candidates, smallest tile first: 64x64 (8 stages), 128x64
// (6 stages), 96x128 (3 stages), 128x128 (3 stages).
static const int kOneRound[] = {22, 21, 15, 4};

template <int NC>
static int pick(const Candidate (&cands)[NC], int M, int N) {
  const int cus = device_cus();
  int best = cands[0].cfg;
  double best_score = -1.0;
  for (const Candidate &c : cands) {
    const TileCfg &t = kTileCfgs[c.cfg];
    const long tiles = (long)((N + t.bn - 1) / t.bn) * ((M + t.bm - 1) / t.bm);
    const long slots = (long)cus * c.slots_per_cu;
    const long rounds = (tiles + slots - 1) / slots;
    const double score = c.quality * (double)tiles / (double)(rounds * slots);
    if (score > best_score) {
      best_score = score;
      best = c.cfg;
    }
  }
  return best;
}

// ZQ_DECODE=<kind> forces the decode kernel (tuning aid): 0 skinny,
// 2 stream, 3 gemv (each only where it applies).
static int forced_decode() {
  static int v = [] {
    const char *e = getenv("ZQ_DECODE");
    return e ? atoi(e) : -1;
  }();
  return v;
}

static int forced_stream() {
  static int v = [] {
    const char *e = getenv("ZQ_STREAM");
    return e ? atoi(e) : 0;
  }();
  return v;
}

static int forced_gemv() {
  static int v = [] {
    const char *e = getenv("ZQ_GEMV");
    return e ? atoi(e) : -1;
  }();
  return v;
}

static Plan choose(int M, int N, int K, int bits) {
  const int f = forced_tile();
  if (f >= 0) return Plan{kTiled, 0, f};
  Plan tp;
  if (sched_lookup(M, N, K, bits, &tp)) return tp;
  if (M <= 64) {
    const int fd = forced_decode();
    const int ldw = bits == 4 ? K / 2 : K;
    const bool gemv_ok = M == 1 && ldw % 1024 == 0;
    const bool stream_ok = M <= 16 && (N & 1) == 0;
    const bool stream17_ok = (N & 1) == 0;
    if (fd == 0) return Plan{kSkinny, (M + 15) / 16, 0};
    if (fd == 2 && stream17_ok) return Plan{kStream, stream_mx(M), 0};
    if (gemv_ok) return Plan{kGemv, 1, 0};
    if (stream_ok) return Plan{kStream, stream_mx(M), 0};
    // 17 .. 64 tokens: W8 over N >= 8192 with more than 32 tokens: 64-row
    // weight tiles with the activations staged once per tile in LDS and an
    // 8-deep copy ring (GPT-J QKV at 64 tokens 17.9 us against 25.3 us for
    // a 64-token ring); otherwise the streaming rings of 32 or 64 token
    // rows (64 x 4096 x 4096 13.9 -> 10.4 us, 64 x 6144 x 24576 W4
    // 100.6 -> 43.8 us against the skinny kernel, which re-reads the whole
    // activation block for every 16 weight rows); odd N: skinny
    if (fd < 0 && (N + 63) / 64 >= 128 && (bits == 8 && M > 32 || !stream17_ok))
      return Plan{kTiled, 0, 22};
    if (stream17_ok) return Plan{kStream, stream_mx(M), 0};
    return Plan{kSkinny, (M + 15) / 16, 0};
  }
  const int cus = device_cus();
  for (int c : kOneRound) {
    const TileCfg &t = kTileCfgs[c];
    const long tiles = (long)((N + t.bn - 1) / t.bn) * ((M + t.bm - 1) / t.bm);
    if (tiles <= cus) return Plan{kTiled, 0, c};
  }
  if (bits == 4 && K < 4096) return Plan{kTiled, 0, 0};
  // packed W4 over wide N with long K (GPT-NeoX-20B FFN1, 2048 x 24576 x
  // 6144): the persistent ping-pong kernel, 302 us against 311 us for
  // 192x256 and 326 us for 256x256 tiles (interleaved repeats; NeoX FFN2,
  // N = 6144, stays faster on 192x256 tiles: 289 against 311 us)
  if (bits == 4 && N >= 16384 && N % 256 == 0 && K % 128 == 0)
    return Plan{kTiled, 0, 28};
  return Plan{kTiled, 0, pick(kW8Candidates, M, N)};
}

// Skinny configurations {BN, NW, U} per 16-token fragment count (tuning
// aid: ZQ_SKINNY=<index> forces one).
static int forced_skinny() {
  static int v = [] {
    const char *e = getenv("ZQ_SKINNY");
    return e ? atoi(e) : -1;
  }();
  return v;
}

template <int MF, bool W4, bool RAW>
static hipError_t run_skinny_mf(int id, const GemmArgs &a, hipStream_t s) {
  switch (id) {
    case 1: return run_skinny<Skinny<16, MF, 8, 8, W4>, RAW>(a, s);
    case 2: return run_skinny<Skinny<16, MF, 16, 4, W4>, RAW>(a, s);
    case 3: return run_skinny<Skinny<32, MF, 8, 4, W4>, RAW>(a, s);
    case 4: return run_skinny<Skinny<16, MF, 4, 4, W4>, RAW>(a, s);
    case 5: return run_skinny<Skinny<32, MF, 16, 2, W4>, RAW>(a, s);
    default: return run_skinny<Skinny<16, MF, 8, (MF <= 2 ? 4 : 2), W4>, RAW>(a, s);
  }
}

template <bool W4, bool RAW>
static hipError_t run(const Plan &pl, const GemmArgs &a, hipStream_t s) {
  if (pl.kind == kGemv) {
    // activation row in LDS when it fits in 8 KB (2 pieces per thread) or
    // 32 KB (8 pieces)
    const int xcls = a.K <= 8192 ? 1 : (a.K <= 32768 ? 2 : 0);
    // default: pieces by rows, activation row in LDS, 6 pieces in flight
    // (ZQ_GEMV=<bits> overrides: 1 interleave, 2 LDS activations, 4 U=6)
    const int f = forced_gemv() >= 0 ? forced_gemv() : 6;
    const int il = f & 1;
    const int xsel = ((f >> 1) & 1) * xcls;
    const int u6 = (f >> 2) & 1;
    if (xsel == 1) {
      if (u6) return run_gemv<Gemv<4, 6, W4, 2>, RAW>(a, s, 2, il);
      return run_gemv<Gemv<4, 8, W4, 2>, RAW>(a, s, 2, il);
    }
    if (xsel == 2) {
      if (u6) return run_gemv<Gemv<4, 6, W4, 8>, RAW>(a, s, 2, il);
      return run_gemv<Gemv<4, 8, W4, 8>, RAW>(a, s, 2, il);
    }
    if (u6) return run_gemv<Gemv<4, 6, W4, 0>, RAW>(a, s, 2, il);
    return run_gemv<Gemv<4, 8, W4, 0>, RAW>(a, s, 2, il);
  }
  if (pl.kind == kStream && !RAW && a.bias && ((uintptr_t)a.bias & 3)) {
    // The rings gather bias pairs as 4-byte words with their copies; a bias
    // that is only 2-byte aligned (a view such as b[1:]) goes to the skinny
    // kernel, which reads it per element.  (A per-element load in the ring
    // epilogue would wait for every copy in flight: vmcnt is in order.)
    return run<W4, RAW>(Plan{kSkinny, (a.M + 15) / 16, 0}, a, s);
  }
  if (pl.kind == kStream) {
    if (pl.mf == 1) return run_stream<Stream<1, 1, 4, 512, 4, W4>, RAW>(a, s);
    if (pl.mf > 16) {
      // 17 .. 64 tokens: 16-row blocks while they number at most one per
      // CU, else 32-row blocks (64 x 6144 x 6144: 23.0 -> 20.5 us; 64 x
      // 6144 x 24576 W4: 67.0 -> 43.8 us); the activation bytes per chunk
      // grow with the token rows, so the chunks shrink to keep the ring in
      // LDS
      const bool fn1 = (a.N + 15) / 16 <= device_cus();
      if constexpr (W4) {
        if (pl.mf == 32)
          return fn1 ? run_stream<Stream<1, 32, 4, 128, 3, W4>, RAW>(a, s)
                     : run_stream<Stream<2, 32, 4, 64, 4, W4>, RAW>(a, s);
        return fn1 ? run_stream<Stream<1, 64, 4, 64, 3, W4>, RAW>(a, s)
                   : run_stream<Stream<2, 64, 4, 64, 3, W4>, RAW>(a, s);
      } else {
        if (pl.mf == 32)
          return fn1 ? run_stream<Stream<1, 32, 4, 128, 4, W4>, RAW>(a, s)
                     : run_stream<Stream<2, 32, 4, 128, 3, W4>, RAW>(a, s);
        return fn1 ? run_stream<Stream<1, 64, 4, 128, 3, W4>, RAW>(a, s)
                   : run_stream<Stream<2, 64, 4, 64, 3, W4>, RAW>(a, s);
      }
    }
    if (forced_stream() == 0) {
      // resident activations (see stream_resident): the ring holds weights
      // only, so it runs deeper with the smaller resident region
      const int xr = stream_resident(a.M, a.N, a.K, a.bits);
      if (xr == 2)
        return run_stream<Stream<W4 ? 2 : 1, 16, 4, W4 ? 256 : 512, 2, W4, false, 2>,
                          RAW>(a, s);
      if (xr == 6)
        return run_stream<Stream<W4 ? 2 : 1, 16, 4, W4 ? 128 : 256, 3, W4, false, 6>,
                          RAW>(a, s);
    }
    // {FN, MX, NW, CK, D}; ZQ_STREAM=<index> picks another ring shape
    // (tuning aid)
    const int v = forced_stream();
    if constexpr (W4) {
      // packed W4 moves two activation bytes per weight byte: 32-row
      // blocks halve that, and measured fastest (NeoX FFN1 / FFN2 at 16
      // tokens: 27.3 -> 22.1 us, 30.7 -> 25.0 us)
      switch (v) {
        case 1: return run_stream<Stream<1, 16, 4, 256, 3, W4>, RAW>(a, s);
        case 2: return run_stream<Stream<1, 16, 4, 128, 6, W4>, RAW>(a, s);
        case 3: return run_stream<Stream<2, 16, 4, 64, 8, W4>, RAW>(a, s);
        default: return run_stream<Stream<2, 16, 4, 128, 4, W4>, RAW>(a, s);
      }
    } else {
      switch (v) {
        case 1: return run_stream<Stream<2, 16, 4, 128, 6, W4>, RAW>(a, s);
        case 2: return run_stream<Stream<2, 16, 4, 256, 3, W4>, RAW>(a, s);
        case 3: return run_stream<Stream<1, 16, 4, 128, 8, W4>, RAW>(a, s);
        default:
          // 32-row blocks when 16-row blocks would outnumber the CUs and
          // 32-row blocks would not (NeoX attention output, 16 x 6144 x
          // 6144: 11.5 -> 10.0 us; with more blocks than CUs either way,
          // 16-row blocks stay: GPT-J QKV 13.3 us against 14.1 us)
          if (stream_w8_wide(a.N))
            return run_stream<Stream<2, 16, 4, 256, 3, W4>, RAW>(a, s);
          return run_stream<Stream<1, 16, 4, 256, 4, W4>, RAW>(a, s);
      }
    }
  }
  if (pl.kind == kSkinny) {
    const int id = forced_skinny();
    switch (pl.mf) {
      case 1: return run_skinny_mf<1, W4, RAW>(id, a, s);
      case 2: return run_skinny_mf<2, W4, RAW>(id, a, s);
      case 3: return run_skinny_mf<3, W4, RAW>(id, a, s);
      default: return run_skinny_mf<4, W4, RAW>(id, a, s);
    }
  }
  return run_tile_cfg<W4, RAW>(pl.cfg, a, s);
}

static hipError_t run_plan(const Plan &pl, const GemmArgs &a, hipStream_t s) {
  if (a.bits == 4)
    return a.raw_i32 ? run<true, true>(pl, a, s) : run<true, false>(pl, a, s);
  return a.raw_i32 ? run<false, true>(pl, a, s) : run<false, false>(pl, a, s);
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t s) {
  return run_plan(choose(a.M, a.N, a.K, a.bits), a, s);
}

// ---------------------------------------------- token quantization on load
// The linear of an fp16 activation x (a.qx holds its bytes): the codes and
// scale of the token-wise quantizer, then the GEMM with its epilogue.  Where
// the plan is the one-token GEMV with the row in LDS, one kernel does both
// (Gemv XQ) and writes the codes and scale for the caller; otherwise the
// row quantizer writes them and the plan's kernel reads them.  Returns the
// activation-row class of the one-kernel form (1: up to 8192 k, 2: up to
// 32768 k), 0 where the two launches run.
static int xq_one_kernel(int M, int N, int K, int bits) {
  if (M != 1 || choose(M, N, K, bits).kind != kGemv) return 0;
  const int f = forced_gemv() >= 0 ? forced_gemv() : 6;
  if (!((f >> 1) & 1)) return 0;  // row not held in LDS
  return K <= 8192 ? 1 : (K <= 32768 ? 2 : 0);
}

// Every block of the one-kernel form quantizes the whole row, so two 4-wave
// blocks per compute unit do that work twice per unit, one 8-wave block once
// (the same waves per SIMD).  One 8-wave block per unit for W4 (whose inner
// loop is heavier in VALU work) and for rows of up to 8192 k: GPT-NeoX-20B
// FFN2 (W4, 6144 x 24576) 16.8 -> 15.9 us, GPT-J attn-out (4096 x 4096)
// 5.8 -> 5.65 us; two 4-wave blocks for longer W8 rows (GPT-J FFN2,
// 4096 x 16384: 13.8 against 14.0 us).  Tuning aid: ZQ_XQ_NW=4 or 8.
static int forced_xq_nw() {
  static int v = [] {
    const char *e = getenv("ZQ_XQ_NW");
    return e ? atoi(e) : -1;
  }();
  return v;
}

static int xq_waves(int bits, int xc) {
  const int f = forced_xq_nw();
  if (f == 4 || f == 8) return f;
  return bits == 4 || xc == 1 ? 8 : 4;
}

hipError_t launch_gemm_xq(const GemmArgs &a, int8_t *qx, float *sx,
                          hipStream_t s) {
  const int xc = xq_one_kernel(a.M, a.N, a.K, a.bits);
  if (xc) {
    const int f = forced_gemv() >= 0 ? forced_gemv() : 6;
    const int il = f & 1;
    if (xq_waves(a.bits, xc) == 8) {
      if (a.bits == 4) {
        if (xc == 1)
          return run_gemv<Gemv<8, 6, true, 1, false, true>, false>(a, s, 1, il, qx, sx);
        return run_gemv<Gemv<8, 6, true, 4, false, true>, false>(a, s, 1, il, qx, sx);
      }
      if (xc == 1)
        return run_gemv<Gemv<8, 6, false, 1, false, true>, false>(a, s, 1, il, qx, sx);
      return run_gemv<Gemv<8, 6, false, 4, false, true>, false>(a, s, 1, il, qx, sx);
    }
    if (a.bits == 4) {
      if (xc == 1)
        return run_gemv<Gemv<4, 6, true, 2, false, true>, false>(a, s, 2, il, qx, sx);
      return run_gemv<Gemv<4, 6, true, 8, false, true>, false>(a, s, 2, il, qx, sx);
    }
    if (xc == 1)
      return run_gemv<Gemv<4, 6, false, 2, false, true>, false>(a, s, 2, il, qx, sx);
    return run_gemv<Gemv<4, 6, false, 8, false, true>, false>(a, s, 2, il, qx, sx);
  }
  const hipError_t e = launch_row_quant(a.qx, nullptr, nullptr, 0.0f, a.M,
                                        a.K, false, qx, sx, nullptr, s);
  if (e != hipSuccess) return e;
  GemmArgs b = a;
  b.qx = qx;
  b.sx = sx;
  return launch_gemm(b, s);
}

// ------------------------------------------------------------- split K
// 17 .. 64 tokens over few weight tiles (N up to about 8K): 64x64 tiles
// leave most compute units idle, and the skinny kernel moves four
// activation bytes per weight byte.  With a caller workspace the K range
// is split over SK workgroups per tile (grid y): each writes its exact
// int32 sums to its own M x N plane of the workspace, and a second kernel
// adds the planes and finishes the same epilogue as every other kernel, so
// y is bit-identical to the unsplit call.
static constexpr int kSplitCfg = 22;  // 64x64 tiles, 8-stage ring

static int splitk_factor(int M, int N, int K, int bits) {
  // up to 32 tokens the streaming rings of the plain call are as fast or
  // faster (32 x 6144 x 6144: 13.9 us against 17.0 us split in 2)
  if (M <= 32 || M > 64) return 1;
  const TileCfg &t = kTileCfgs[kSplitCfg];
  const long tiles = (long)((N + t.bn - 1) / t.bn) * ((M + t.bm - 1) / t.bm);
  if (tiles >= 128) return 1;
  const int cus = device_cus();
  for (int sk : {8, 4, 2}) {
    // whole 128-k stages, slices of at least 3072 k and at least 128
    // workgroups: shorter slices or fewer workgroups pay more in prologue,
    // partial stores and the reduction than they gain (K = 4096 in 2 or 4
    // slices measured equal or slower than the plain call; K = 6144 in 2
    // slices and K = 16384 in 4 faster: 64 x 6144 x 6144 20.6 -> 18.8 us,
    // 64 x 4096 x 16384 28.2 -> 23.5 us).  Packed W4 halves the weight
    // bytes per slice, and two slices lose to the W4 ring (48 x 6144 x
    // 6144: 15.5 us against 18.4 us).
    if (K % (sk * 128) == 0 && K / sk >= 3072 && tiles * sk >= 128 &&
        tiles * sk <= cus && (bits == 8 || sk >= 4))
      return sk;
  }
  return 1;
}

size_t gemm_ws_bytes(int M, int N, int K, int bits) {
  if (M <= 0) return 0;
  Plan tp;
  if (forced_tile() >= 0 || sched_lookup(M, N, K, bits, &tp)) return 0;
  const int sk = splitk_factor(M, N, K, bits);
  return sk > 1 ? (size_t)sk * M * N * 4 : 0;
}

// One thread per 4 outputs of a row: the SK partial quads (all loads in
// flight together), then the shared epilogue.
template <int SK>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(GemmArgs p, const int32_t *__restrict__ ws) {
  const int nq = (p.N + 3) / 4;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)p.M * nq) return;
  const int t = (int)(i / nq), nb = (int)(i % nq) * 4;
  const QuadCol qc = load_quad_col(p, nb);
  const float sxt = p.sx[t];
  const size_t plane = (size_t)p.M * p.N;
  const int32_t *src = ws + (size_t)t * p.N + nb;
  v4i part[SK];
  if ((p.N & 3) == 0) {
#pragma unroll
    for (int z = 0; z < SK; ++z)
      part[z] = *reinterpret_cast<const v4i *>(src + z * plane);
  } else {
#pragma unroll
    for (int z = 0; z < SK; ++z)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[z][r] = nb + r < p.N ? src[z * plane + r] : 0;
  }
  v4i a = part[0];
#pragma unroll
  for (int z = 1; z < SK; ++z) a += part[z];
  store_quad<false, false>(p, t, nb, a, sxt, qc);
}

hipError_t launch_gemm_ws(const GemmArgs &a, void *ws, hipStream_t s) {
  Plan tp;
  const int sk = (forced_tile() >= 0 || sched_lookup(a.M, a.N, a.K, a.bits, &tp))
                     ? 1
                     : splitk_factor(a.M, a.N, a.K, a.bits);
  if (sk <= 1 || a.raw_i32) return launch_gemm(a, s);
  GemmArgs r = a;
  r.out = ws;
  r.raw_i32 = true;
  using C8 = Tile<64, 64, 32, 32, 8, false>;
  using C4 = Tile<64, 64, 32, 32, 8, true>;
  const int tiles = ((a.N + 63) / 64) * ((a.M + 63) / 64);
  if (a.bits == 4)
    hipLaunchKernelGGL((gemm_tiled_kernel<C4, true>), dim3(tiles, sk),
                       dim3(C4::NT), 0, s, r);
  else
    hipLaunchKernelGGL((gemm_tiled_kernel<C8, true>), dim3(tiles, sk),
                       dim3(C8::NT), 0, s, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long quads = (long)a.M * ((a.N + 3) / 4);
  const dim3 grid((unsigned)((quads + 255) / 256));
  const int32_t *w32 = static_cast<const int32_t *>(ws);
  if (sk == 2)
    hipLaunchKernelGGL(splitk_reduce_kernel<2>, grid, dim3(256), 0, s, a, w32);
  else if (sk == 4)
    hipLaunchKernelGGL(splitk_reduce_kernel<4>, grid, dim3(256), 0, s, a, w32);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<8>, grid, dim3(256), 0, s, a, w32);
  return hipGetLastError();
}

int describe_gemm_ws_plan(int M, int N, int K, int bits, char *buf, int len) {
  Plan tp;
  const int sk = (forced_tile() >= 0 || sched_lookup(M, N, K, bits, &tp))
                     ? 1
                     : splitk_factor(M, N, K, bits);
  if (sk <= 1) return describe_gemm_plan(M, N, K, bits, buf, len);
  return snprintf(buf, len,
                  "splitk SK=%d tiled cfg=%d BN=64 BM=64 W%d tiles=%d + reduce",
                  sk, kSplitCfg, bits, ((N + 63) / 64) * ((M + 63) / 64) * sk);
}

// ------------------------------------------------------------- tuner
static const char *kind_name(PlanKind k) {
  switch (k) {
    case kGemv: return "gemv";
    case kStream: return "stream";
    case kSkinny: return "skinny";
    case kTiled: return "tiled";
  }
  return "?";
}

static bool kind_from_name(const char *s, PlanKind *k) {
  static const PlanKind all[] = {kGemv, kStream, kSkinny, kTiled};
  for (PlanKind c : all)
    if (strcmp(s, kind_name(c)) == 0) {
      *k = c;
      return true;
    }
  return false;
}

unsigned sched_generation() { return g_sched_gen.load(); }

void sched_clear() {
  std::lock_guard<std::mutex> lk(g_sched_mu);
  g_sched.clear();
  g_sched_gen++;
}

int sched_entries() {
  std::lock_guard<std::mutex> lk(g_sched_mu);
  return (int)g_sched.size();
}

// One line per entry: "<bits> <N> <K> <M lo> <M hi> <kind> <tile cfg>".
size_t sched_export(char *buf, size_t len) {
  std::string out;
  {
    std::lock_guard<std::mutex> lk(g_sched_mu);
    std::vector<SchedEntry> v = g_sched;
    std::sort(v.begin(), v.end(), [](const SchedEntry &x, const SchedEntry &y) {
      if (x.bits != y.bits) return x.bits < y.bits;
      if (x.N != y.N) return x.N < y.N;
      if (x.K != y.K) return x.K < y.K;
      return x.mlo < y.mlo;
    });
    char line[96];
    for (const SchedEntry &e : v) {
      snprintf(line, sizeof line, "%d %d %d %d %d %s %d\n", e.bits, e.N, e.K,
               e.mlo, e.mhi, kind_name(e.kind), e.kind == kTiled ? e.cfg : 0);
      out += line;
    }
  }
  if (buf && len > 0) {
    const size_t n = out.size() < len - 1 ? out.size() : len - 1;
    memcpy(buf, out.data(), n);
    buf[n] = '\0';
  }
  return out.size() + 1;
}

// Parses the whole text first; nothing is applied unless every line is a
// valid entry.  Returns the number of entries, or -(line number) of the
// first bad line.
int sched_import(const char *text) {
  std::vector<SchedEntry> add;
  int lineno = 0;
  const char *p = text;
  while (*p) {
    const char *e = strchr(p, '\n');
    const size_t n = e ? (size_t)(e - p) : strlen(p);
    ++lineno;
    std::string line(p, n);
    p += n + (e ? 1 : 0);
    const size_t h = line.find('#');
    if (h != std::string::npos) line.resize(h);
    if (line.find_first_not_of(" \t\r") == std::string::npos) continue;
    SchedEntry s{};
    char kind[16];
    int used = 0;
    if (sscanf(line.c_str(), "%d %d %d %d %d %15s %d %n", &s.bits, &s.N, &s.K,
               &s.mlo, &s.mhi, kind, &s.cfg, &used) != 7 ||
        line.find_first_not_of(" \t\r", used) != std::string::npos)
      return -lineno;
    if ((s.bits != 8 && s.bits != 4) || s.N <= 0 || s.K <= 0 || s.K % 64 != 0 ||
        s.mlo < 1 || s.mhi < s.mlo || !kind_from_name(kind, &s.kind))
      return -lineno;
    // the plan must apply at both ends of its range (and so in between)
    if (!plan_applies(s.kind, s.cfg, s.mlo, s.N, s.K, s.bits) ||
        !plan_applies(s.kind, s.cfg, s.mhi, s.N, s.K, s.bits))
      return -lineno;
    if (s.kind != kTiled) s.cfg = 0;
    add.push_back(s);
  }
  std::lock_guard<std::mutex> lk(g_sched_mu);
  for (const SchedEntry &s : add) sched_put_locked(s);
  g_sched_gen++;
  return (int)add.size();
}

// Every plan that applies to (M, N, K, bits).
static std::vector<Plan> candidates(int M, int N, int K, int bits) {
  std::vector<Plan> v;
  for (PlanKind k : {kGemv, kStream, kSkinny})
    if (plan_applies(k, 0, M, N, K, bits)) v.push_back(make_plan(k, 0, M, false));
  for (int c = 0; c < kNumTileCfgs; ++c)
    if (plan_applies(kTiled, c, M, N, K, bits)) v.push_back(make_plan(kTiled, c, M, false));
  return v;
}

// Times every applicable plan at each M of ms[] (ascending) on the caller's
// buffers (sized for the largest M) and records the fastest for the range
// (previous M, M].  Synchronizes the stream; not for use under capture.
hipError_t tune_gemm(const GemmArgs &base, const int *ms, int nm, int reps,
                     hipStream_t s, int *chosen_kind, int *chosen_cfg,
                     float *chosen_us) {
  hipEvent_t e0, e1;
  hipError_t err = hipEventCreate(&e0);
  if (err != hipSuccess) return err;
  err = hipEventCreate(&e1);
  if (err != hipSuccess) {
    (void)hipEventDestroy(e0);
    return err;
  }
  std::vector<SchedEntry> found;
  int prev = 0;
  for (int i = 0; i < nm && err == hipSuccess; ++i) {
    GemmArgs a = base;
    a.M = ms[i];
    // two passes over the candidates, each keeping its faster pass, so that
    // a clock or power transient during one timing does not decide
    const std::vector<Plan> cands = candidates(a.M, a.N, a.K, a.bits);
    std::vector<float> t(cands.size(), 0.0f);
    for (int pass = 0; pass < 2 && err == hipSuccess; ++pass)
      for (size_t c = 0; c < cands.size() && err == hipSuccess; ++c) {
        const Plan &pl = cands[c];
        err = run_plan(pl, a, s);  // warm-up (and code-object load)
        if (err == hipSuccess) err = hipEventRecord(e0, s);
        for (int r = 0; r < reps && err == hipSuccess; ++r) err = run_plan(pl, a, s);
        if (err == hipSuccess) err = hipEventRecord(e1, s);
        if (err == hipSuccess) err = hipEventSynchronize(e1);
        float ms_ = 0.0f;
        if (err == hipSuccess) err = hipEventElapsedTime(&ms_, e0, e1);
        const float us = 1e3f * ms_ / reps;
        if (pass == 0 || us < t[c]) t[c] = us;
      }
    if (err != hipSuccess) break;
    size_t bi = 0;
    for (size_t c = 1; c < cands.size(); ++c)
      if (t[c] < t[bi]) bi = c;
    const Plan bp = cands[bi];
    const float best = t[bi];
    found.push_back(SchedEntry{a.bits, a.N, a.K, prev + 1, a.M, bp.kind,
                               bp.kind == kTiled ? bp.cfg : 0});
    if (chosen_kind) chosen_kind[i] = (int)bp.kind;
    if (chosen_cfg) chosen_cfg[i] = bp.kind == kTiled ? bp.cfg : -1;
    if (chosen_us) chosen_us[i] = best;
    prev = a.M;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lk(g_sched_mu);
  for (const SchedEntry &e : found) sched_put_locked(e);
  g_sched_gen++;
  return hipSuccess;
}

// ---------------------------------------------------- quantized output
// The GEMM's fp16 output in the workspace, then the token quantizer over
// it: the same kernels as the unfused pair of calls.  (Quantizing in the
// GEMM epilogue needs every column tile of a token row finished before any
// of its codes: a grid-wide barrier, whose cost on this device is larger
// than the fp16 round trip it would save.)
size_t gemm_quant_ws_bytes(int M, int N) { return (size_t)M * N * 2; }

hipError_t launch_gemm_quant(const GemmArgs &a, int8_t *qy, float *sy,
                             void *ws, hipStream_t s) {
  GemmArgs g = a;
  g.out = ws;
  g.raw_i32 = false;
  const hipError_t e = launch_gemm(g, s);
  if (e != hipSuccess) return e;
  return launch_row_quant(ws, nullptr, nullptr, 0.0f, a.M, a.N, false, qy, sy,
                          nullptr, s);
}

// ------------------------------------------------ fp16 activations (W8A16)
// INT8 weights with fp16 activations (qx points at fp16 [M][K]; sx unused):
// the tiled kernel with A16 tiles.  {BN, BM, WN, WM, stages}.
struct A16Cfg {
  int bn, bm, wn, wm, s;
};
static const A16Cfg kA16Cfgs[] = {
    {256, 256, 64, 64, 3},  // 0: 16 waves, 48 KB stages
    {128, 128, 64, 64, 3},  // 1: 4 waves
    {64, 64, 32, 32, 10},   // 2: 4 waves, decode-sized M
    {192, 256, 64, 64, 3},  // 3: 12 waves
    {128, 64, 64, 32, 8},   // 4: 4 waves
};
constexpr int kNumA16Cfgs = sizeof(kA16Cfgs) / sizeof(kA16Cfgs[0]);

// ZQ_A16_TILE=<index> forces one configuration (tuning aid).
static int forced_a16() {
  static int v = [] {
    const char *e = getenv("ZQ_A16_TILE");
    if (!e) return -1;
    const int i = atoi(e);
    return (i >= 0 && i < kNumA16Cfgs) ? i : -1;
  }();
  return v;
}

// From measured sweeps (GPT-NeoX20B QKV and out shapes): decode-sized M on
// 128x64 tiles with an 8-deep ring; prefill on 192x256 tiles, or 128x128
// when 192x256 would leave most compute units idle.
static int choose_a16(int M, int N) {
  const int f = forced_a16();
  if (f >= 0) return f;
  if (M <= 64) return 4;
  const long t = (long)((N + 191) / 192) * ((M + 255) / 256);
  return t >= 128 ? 3 : 1;
}

static bool a16_gemv(int M, int K) {
  return forced_a16() < 0 && M == 1 && K % 1024 == 0 && K <= 32768;
}

// ZQ_A16_STREAM=<index> picks the stream configuration for up to 16 tokens
// (tuning aid).
static int a16_stream_cfg() {
  static int v = [] {
    const char *e = getenv("ZQ_A16_STREAM");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// Up to 64 tokens with even N (bias pairs): the streaming kernel, except
// more than 32 tokens over N >= 8192, where the 128x64 tiles are faster
// (64 x 18432 x 6144: 77.9 us against 90.6 us for a 64-row ring).  Against
// those tiles elsewhere: 32 x 4096 x 4096 53.5 -> 11.3 us, 48 x 6144 x 6144
// 74.8 -> 37.0 us, 24 x 18432 x 6144 76.9 -> 54.1 us.
static bool a16_stream(int M, int N, int K) {
  return forced_a16() < 0 && !a16_gemv(M, K) && M >= 1 && M <= 64 &&
         (N & 1) == 0 && !(M > 32 && N >= 8192);
}

hipError_t launch_gemm_w8a16(const GemmArgs &a, hipStream_t s) {
  if (a16_gemv(a.M, a.K)) {
    // one token: weight rows streamed in 1 KB pieces, the fp16 activation
    // row (up to 16 KB, else 64 KB) in LDS, whole rows per wave
    if (a.K <= 8192) return run_gemv<Gemv<4, 6, false, 4, true>, false>(a, s, 2, 0);
    return run_gemv<Gemv<4, 6, false, 16, true>, false>(a, s, 2, 0);
  }
  // the rings gather bias pairs as 4-byte words: a bias that is only 2-byte
  // aligned takes the tiles, which read it per element
  const bool bias2 = a.bias && ((uintptr_t)a.bias & 3);
  if (a16_stream(a.M, a.N, a.K) && !bias2) {
    if (a.M == 1) return run_stream<Stream<1, 1, 4, 512, 4, false, true>, false>(a, s);
    if (a.M > 16) {
      // 17 .. 64 tokens: the per-wave fp32 partials and the activation
      // bytes grow with the token rows, so the chunks shrink to keep the
      // ring in LDS; 32-row blocks once 16-row blocks outnumber the CUs
      // (up to 32 tokens; a 64-row ring of 32-row blocks does not fit)
      if (a.M > 32) return run_stream<Stream<1, 64, 4, 64, 3, false, true>, false>(a, s);
      if ((a.N + 15) / 16 <= device_cus())
        return run_stream<Stream<1, 32, 4, 128, 3, false, true>, false>(a, s);
      return run_stream<Stream<2, 32, 4, 64, 3, false, true>, false>(a, s);
    }
    // {FN, MX, NW, CK, D}; the default (32-row blocks, 128-byte chunks,
    // 4-deep rings) measured fastest on NeoX QKV at 16 tokens (2.83 TB/s,
    // against 2.3 - 2.6 for the others)
    switch (a16_stream_cfg()) {
      case 1: return run_stream<Stream<1, 16, 4, 128, 6, false, true>, false>(a, s);
      case 2: return run_stream<Stream<1, 16, 4, 256, 3, false, true>, false>(a, s);
      case 3: return run_stream<Stream<1, 16, 4, 128, 5, false, true>, false>(a, s);
      default: return run_stream<Stream<2, 16, 4, 128, 4, false, true>, false>(a, s);
    }
  }
  switch (choose_a16(a.M, a.N)) {
    case 0: return run_tiled<Tile<256, 256, 64, 64, 3, false, 128, true>, false>(a, s);
    case 1: return run_tiled<Tile<128, 128, 64, 64, 3, false, 128, true>, false>(a, s);
    case 2: return run_tiled<Tile<64, 64, 32, 32, 10, false, 128, true>, false>(a, s);
    case 3: return run_tiled<Tile<192, 256, 64, 64, 3, false, 128, true>, false>(a, s);
    default: return run_tiled<Tile<128, 64, 64, 32, 8, false, 128, true>, false>(a, s);
  }
}

int describe_gemm_w8a16_plan(int M, int N, int K, char *buf, int len) {
  if (a16_gemv(M, K))
    return snprintf(buf, len, "gemv-a16 NW=4 U=6 rows=%d x_in_lds=1", N);
  if (a16_stream(M, N, K)) {
    const int cfg = M == 1 || M > 16 ? 0 : a16_stream_cfg();
    const int mx = M == 1 ? 1 : M <= 16 ? 16 : M <= 32 ? 32 : 64;
    const int bn = mx > 16 ? (mx == 32 && (N + 15) / 16 > device_cus() ? 32 : 16)
                           : (M > 1 && cfg == 0) ? 32 : 16;
    return snprintf(buf, len, "stream-a16 MX=%d NW=4 cfg=%d BN=%d row_blocks=%d",
                    mx, cfg, bn, (N + bn - 1) / bn);
  }
  const int i = choose_a16(M, N);
  const A16Cfg &c = kA16Cfgs[i];
  return snprintf(buf, len,
                  "tiled-a16 cfg=%d BN=%d BM=%d WN=%d WM=%d stages=%d tiles=%d", i,
                  c.bn, c.bm, c.wn, c.wm, c.s,
                  ((N + c.bn - 1) / c.bn) * ((M + c.bm - 1) / c.bm));
}

int describe_gemm_plan(int M, int N, int K, int bits, char *buf, int len) {
  const Plan pl = choose(M, N, K, bits);
  const char *src = pl.tuned ? " [table]" : "";
  if (pl.kind == kGemv) {
    // the launch grid of run_gemv with two blocks per CU
    int grid = 2 * device_cus();
    if (grid > N) grid = N;
    int rpb = (N + grid - 1) / grid;
    if (rpb > 1024) rpb = 1024;
    grid = (N + rpb - 1) / rpb;
    return snprintf(buf, len, "gemv NW=4 U=6 W%d rows=%d x_in_lds=%d grid=%d%s",
                    bits, N, K <= 32768 ? 1 : 0, grid, src);
  }
  if (pl.kind == kStream) {
    const int xr = pl.mf == 16 && forced_stream() == 0
                       ? stream_resident(M, N, K, bits) : 0;
    const int bn = xr ? (bits == 4 ? 32 : 16)
                   : pl.mf > 16 ? ((N + 15) / 16 <= device_cus() ? 16 : 32)
                   : (pl.mf > 1 && forced_stream() == 0 &&
                      (bits == 4 || stream_w8_wide(N))) ? 32 : 16;
    const int nrb = (N + bn - 1) / bn;
    return snprintf(buf, len,
                    "stream BN=%d MX=%d NW=4 W%d%s row_blocks=%d grid=%d%s", bn,
                    pl.mf, bits, xr ? (xr == 2 ? " xres=2" : " xres=6") : "",
                    nrb, nrb < device_cus() ? nrb : device_cus(), src);
  }
  if (pl.kind == kSkinny)
    return snprintf(buf, len, "skinny BN=16 MF=%d NW=8 U=%d W%d blocks=%d%s",
                    pl.mf, pl.mf <= 2 ? 4 : 2, bits, (N + 15) / 16, src);
  const TileCfg &c = kTileCfgs[pl.cfg];
  const int tiles = ((N + c.bn - 1) / c.bn) * ((M + c.bm - 1) / c.bm);
  const int kps = c.kb;  // k per stage (INT8 activations)
  if (c.persist && N % c.bn == 0 && K % kps == 0 && K / kps >= c.s)
    return snprintf(buf, len,
                    "tiled cfg=%d BN=%d BM=%d WN=%d WM=%d stages=%d kb=%d W%d "
                    "tiles=%d %s grid=%d%s",
                    pl.cfg, c.bn, c.bm, c.wn, c.wm, c.s, c.kb, bits, tiles,
                    "persistent ping-pong",
                    tiles < device_cus() ? tiles : device_cus(), src);
  return snprintf(buf, len,
                  "tiled cfg=%d BN=%d BM=%d WN=%d WM=%d stages=%d kb=%d W%d tiles=%d%s",
                  pl.cfg, c.bn, c.bm, c.wn, c.wm, c.s, c.kb, bits, tiles, src);
}

int describe_gemm_xq_plan(int M, int N, int K, int bits, char *buf, int len) {
  if (const int xc = xq_one_kernel(M, N, K, bits)) {
    // the launch grid of run_gemv: one 8-wave or two 4-wave blocks per CU
    const int nw = xq_waves(bits, xc);
    int grid = (nw == 8 ? 1 : 2) * device_cus();
    if (grid > N) grid = N;
    int rpb = (N + grid - 1) / grid;
    if (rpb > 1024) rpb = 1024;
    grid = (N + rpb - 1) / rpb;
    return snprintf(buf, len,
                    "quantize-on-load gemv NW=%d U=6 W%d rows=%d x_in_lds=1 "
                    "grid=%d", nw, bits, N, grid);
  }
  const int w = snprintf(buf, len, "row-quant + ");
  return w + describe_gemm_plan(M, N, K, bits, buf + w, len - w);
}

}  // namespace zq
