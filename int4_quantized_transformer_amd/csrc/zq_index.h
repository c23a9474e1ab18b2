// zq_index.h -- launch geometry of the GEMM kernels as plain integer
// arithmetic: the tile / ring configurations and the address of every
// global -> LDS copy, shared by the kernels (zq_gemm.hip) and by the host
// replay that checks those addresses against the buffer bounds for every
// configuration and problem shape (tests/index_replay.cpp, built with the
// host compiler under the address and undefined-behaviour sanitizers).
// The includer defines ZQ_HD: "__host__ __device__" in the library, empty
// for the host replay.
#pragma once

#include <stdint.h>

#ifndef ZQ_HD
#error "define ZQ_HD before including zq_index.h"
#endif

namespace zq {

constexpr int kWave = 64;

// ------------------------------------------------------------ XCD mapping
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Remap the hardware order so that each XCD receives a contiguous
// range of logical tile ids; the map is a bijection on [0, total).
ZQ_HD inline int xcd_remap(int pid, int total) {
  constexpr int X = 8;
  const int q = total / X, r = total % X;
  const int x = pid % X, i = pid / X;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// =================================================================== tiles
// Block tile BN (n) x BM (t), k in stages of KB = 128 activation bytes
// (64 packed W4 bytes), or KB = 64 for W8.  LDS rows are unpadded (128 B, or
// 64 B for packed W4) and their 16-byte chunks are XOR-swizzled so that the
// 16-byte fragment reads of 8 consecutive rows hit 8 different bank groups:
//   128-byte rows: slot = chunk ^ ((row >> 1) & 7)
//    64-byte rows: slot = chunk ^ ((row >> 2) & 3)
template <int BN_, int BM_, int WN_, int WM_, int S_, bool W4_, int KB_ = 128,
          bool A16_ = false>
struct TileGeom {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_, S = S_;
  static constexpr bool W4 = W4_;
  // A16: fp16 activations (2 bytes per k) with INT8 weights, on the fp16
  // MFMA (32x32x16): a stage holds 64 k, rows of 128 activation bytes and 64
  // weight bytes, and k advances 16 per MFMA k-step
  static constexpr bool A16 = A16_;
  static constexpr int KB = KB_, KS = KB_ / 32;     // MFMA k-steps per stage
  static constexpr int KPS = A16 ? KB / 2 : KB;     // k values per stage
  static constexpr int NWN = BN / WN, NWM = BM / WM;
  static constexpr int NWAVES = NWN * NWM, NT = NWAVES * kWave;
  static constexpr int FN = WN / 32, FM = WM / 32;
  static constexpr int XROW = KB;                   // activation bytes/row/stage
  static constexpr int WROW = (W4 || A16) ? KB / 2 : KB;  // weight bytes/row/stage
  static constexpr int WCPR = WROW / 16, XCPR = XROW / 16;  // chunks per row
  static constexpr int WRPI = 64 / WCPR, XRPI = 64 / XCPR;  // rows per wave copy
  static constexpr int WINS = BN / WRPI, XINS = BM / XRPI;  // wave copies/stage
  // copies per wave (the same for every wave, so that every vmcnt wait is a
  // constant); when the waves do not divide the copies evenly the last ones
  // are padding that land in the padded tail of their region, never read
  static constexpr int IW = (WINS + NWAVES - 1) / NWAVES;
  static constexpr int IX = (XINS + NWAVES - 1) / NWAVES;
  static constexpr int WBYTES = IW * NWAVES * 1024;  // weight region (padded)
  static constexpr int XBYTES = IX * NWAVES * 1024;  // activation region
  static constexpr int STAGE = WBYTES + XBYTES;
  // epilogue operands copied into LDS with stage 0: bias of the tile's BN
  // columns and scales of its BM tokens, each padded to whole 256-byte wave
  // copies (64 lanes x 4 bytes)
  static constexpr int AUX_BIAS = ((BN * 2 + 255) / 256) * 256;
  static constexpr int AUX_SX = ((BM * 4 + 255) / 256) * 256;
  static constexpr int LDS = S * STAGE + AUX_BIAS + AUX_SX;
  static constexpr bool ok_width = KB == 128 || (KB == 64 && !W4 && !A16);
  static constexpr bool ok_a16 = !(A16 && W4);
  static constexpr bool ok_split = BN % WRPI == 0 && BM % XRPI == 0;
  static constexpr bool ok_tile = WN % 32 == 0 && WM % 32 == 0 && S >= 2;
  static constexpr bool ok_vmcnt = (IW + IX) * (S - 2) < 64;
  static constexpr bool ok_lds = LDS <= 160 * 1024;
  // whether the configuration is a valid kernel instance (Tile asserts it)
  static constexpr bool ok = ok_width && ok_a16 && ok_split && ok_tile &&
                             ok_vmcnt && ok_lds;
};

template <int BN_, int BM_, int WN_, int WM_, int S_, bool W4_, int KB_ = 128,
          bool A16_ = false>
struct Tile : TileGeom<BN_, BM_, WN_, WM_, S_, W4_, KB_, A16_> {
  using G = TileGeom<BN_, BM_, WN_, WM_, S_, W4_, KB_, A16_>;
  static_assert(G::ok_width, "stage width");
  static_assert(G::ok_a16, "W4 with fp16 activations");
  static_assert(G::ok_split, "copy split");
  static_assert(G::ok_tile, "tile");
  static_assert(G::ok_vmcnt, "vmcnt range");
  static_assert(G::ok_lds, "LDS");
};

ZQ_HD inline int sw128(int row) { return (row >> 1) & 7; }
ZQ_HD inline int sw64(int row) { return (row >> 2) & 3; }

template <int BYTES>
ZQ_HD inline int wswz(int chunk, int row) {
  if constexpr (BYTES == 128) return chunk ^ sw128(row);
  else return chunk ^ sw64(row);
}

// One 16-byte lane copy: byte offset into the operand's global buffer, and
// byte offset of the wave's 1 KB copy within the stage (the lane's bytes go
// to lds + 16 * lane).
struct CopyAddr {
  int64_t goff;
  int lds;
};

// Weight copy q (of IW * NWAVES per stage) of stage kt of the tile whose
// first weight row is n0: rows past the tile or past N re-read a valid row
// (never stored); with K % 128 == 64 the unused upper half of the last
// stage re-reads the lower half.
template <class C>
ZQ_HD inline CopyAddr tile_w_copy(int q, int lane, int n0, int kt, int N,
                                  int ldw) {
  const int row = q * C::WRPI + lane / C::WCPR;  // >= BN: padding copy
  const int chunk = wswz<C::WROW>(lane % C::WCPR, row);
  int n = n0 + (row < C::BN ? row : C::BN - 1);
  n = n < N ? n : N - 1;
  int kb = kt * C::WROW + chunk * 16;
  if (kb >= ldw) kb -= C::WROW / 2;
  return CopyAddr{(int64_t)n * ldw + kb, q * 1024};
}

// Activation copy q (of IX * NWAVES per stage), as tile_w_copy for the
// token rows m0 .. m0 + BM - 1 of x [M][K] (fp16 for A16 tiles).
template <class C>
ZQ_HD inline CopyAddr tile_x_copy(int q, int lane, int m0, int kt, int M,
                                  int K) {
  const int row = q * C::XRPI + lane / C::XCPR;  // >= BM: padding copy
  const int chunk = wswz<C::XROW>(lane % C::XCPR, row);
  int t = m0 + (row < C::BM ? row : C::BM - 1);
  t = t < M ? t : M - 1;
  constexpr int XB = C::A16 ? 2 : 1;              // activation bytes per k
  int kb = kt * C::XROW + chunk * 16;
  if (kb >= K * XB) kb -= C::XROW / 2;
  return CopyAddr{(int64_t)t * K * XB + kb, C::WBYTES + q * 1024};
}

// ---------------------------------------------------------- ping-pong aux
// Epilogue operands of one tile of the persistent kernel, gathered as
// dwords: bias of its BN columns (BN / 2 dwords), scales of its BM tokens,
// the group scale of each 32-column fragment.
template <class C>
struct PAux {
  static constexpr int BIAS = C::BN * 2;
  static constexpr int SX = C::BM * 4;
  static constexpr int SW = (C::BN / 32) * 4;
  static constexpr int DW = (BIAS + SX + SW) / 4;          // dwords per tile
  static constexpr int NCOPY = (DW + 63) / 64;              // wave copies
  static constexpr int BYTES = NCOPY * 256;
  static constexpr int LDS = C::S * C::STAGE + 2 * BYTES;
  static_assert(C::BN % 32 == 0 && LDS <= 160 * 1024, "persistent LDS");
};

// Source of aux dword e of the tile at (n0, m0): which array (0 bias
// dwords, 1 sx, 2 sw, 3 none: a padding lane) and the element index in it.
enum AuxSrc { kAuxBias = 0, kAuxSx = 1, kAuxSw = 2, kAuxPad = 3 };
struct AuxElem {
  int src, index;
};

template <class C>
ZQ_HD inline AuxElem persist_aux_elem(int e, int n0, int m0, int M, int G) {
  using A = PAux<C>;
  if (e < A::BIAS / 4) return AuxElem{kAuxBias, n0 / 2 + e};
  if (e < (A::BIAS + A::SX) / 4) {
    const int t = m0 + e - A::BIAS / 4;
    return AuxElem{kAuxSx, t < M ? t : M - 1};
  }
  if (e < A::DW) {
    const int n = n0 + 32 * (e - (A::BIAS + A::SX) / 4);
    return AuxElem{kAuxSw, n / G};
  }
  return AuxElem{kAuxPad, 0};
}

// Tile of workgroup pid (after xcd_remap) of the tiled kernel: groups of
// GM token tiles that share one weight tile, token tiles fastest (the last
// group may be short).
constexpr int kTileGroup = 4;  // GM of the tiled kernel

template <int GM>
ZQ_HD inline void grouped_tile(int pid, int tiles_m, int tiles_n, int &tm,
                               int &tn) {
  const int per_group = GM * tiles_n;
  const int first_m = (pid / per_group) * GM;
  const int gsz = tiles_m - first_m < GM ? tiles_m - first_m : GM;
  tm = first_m + (pid % per_group) % gsz;
  tn = (pid % per_group) / gsz;
}

// Tile of logical index L of the persistent kernel: groups of (at most) 4
// token tiles, token tiles fastest within a group, then the weight tiles,
// then the next group.  The 32 workgroups of one XCD (contiguous logical
// slots, see xcd_remap) then hold 8 weight tiles x 4 token tiles at a time,
// which is the split of 32 that fetches the fewest operand bytes into the
// XCD's L2 at the prefill shapes (8 token tiles x 4 weight tiles, the order
// without groups, re-fetches every activation row in every round).
ZQ_HD inline void persist_tile(int L, int tiles_m, int tiles_n, int &tm,
                               int &tn) {
  constexpr int TG = 4;
  const int gsize = TG * tiles_n;
  const int grp = L / gsize, r = L - grp * gsize;
  const int first = grp * TG;
  const int gs = tiles_m - first < TG ? tiles_m - first : TG;
  tm = first + r % gs;
  tn = r / gs;
}

// =================================================================== rings
// Decode-sized M: persistent blocks of NW waves over row blocks of BN = 16 FN
// weight rows; each wave streams chunks of CK bytes of every row of a block
// (and the matching activation bytes of MX token rows) through its own ring
// of D LDS slots.
//
// XR > 0 (resident activations): a wave always takes the same chunks of K
// (c = wave, wave + NW, ...), so it copies the activation bytes of at most
// XR such chunks once, into an LDS region of its own, and its ring carries
// only the weights and the epilogue operands of each row block.
template <int FN_, int MX_, int NW_, int CK_, int D_, bool W4_, bool A16_ = false,
          int XR_ = 0>
struct StreamGeom {
  static constexpr int FN = FN_, MX = MX_, NW = NW_, CK = CK_, D = D_;
  static constexpr bool W4 = W4_, A16 = A16_;
  static constexpr int XR = XR_;
  static constexpr int BN = 16 * FN;
  static constexpr int MF = (MX + 15) / 16;
  static constexpr int NT = NW * kWave;
  static constexpr int XCK = (W4 || A16) ? 2 * CK : CK;
  static constexpr int SPC = CK / 64;                // k-steps per chunk
  static constexpr int IW = BN * CK / 1024;          // weight copies
  static constexpr int IXC = (MX * XCK + 1023) / 1024;  // copies per chunk's activations
  static constexpr int IX = XR > 0 ? 0 : IXC;        // activation copies per ring slot
  static constexpr int NAUX = MX + BN + BN / 2;      // aux dwords
  static constexpr int IA = (NAUX + 63) / 64;        // aux copies
  static constexpr int P = IW + IX + IA;             // copies per chunk
  static constexpr int XOFF = IW * 1024, AOFF = (IW + IX) * 1024;
  static constexpr int SLOT = AOFF + IA * 256;
  static constexpr int XCH = IXC * 1024;             // a chunk's activation image
  static constexpr int XRES = XR * XCH;              // resident region per wave
  static constexpr int RED = (A16 ? NW : 1) * FN * MF * 1024;  // one half
  static constexpr int LDS = NW * (D * SLOT + XRES) + 2 * RED;
  static constexpr int WSW = (CK / 16 < 16 ? CK / 16 : 16) - 1;
  static constexpr int XSW = (XCK / 16 < 16 ? XCK / 16 : 16) - 1;
  static constexpr bool ok_a16 = !(W4 && A16);
  static constexpr bool ok_chunk = CK % 64 == 0 && (BN * CK) % 1024 == 0;
  // the resident copies are issued before the ring's first chunks (older,
  // so complete once the first chunk is) and stay below the counter range
  static constexpr bool ok_vmcnt = D >= 2 && XR * IXC + (D - 1) * P < 64;
  static constexpr bool ok_lds = LDS <= 160 * 1024;
  static constexpr bool ok_xr = XR == 0 || (!A16 && MX <= 16);
  // whether the configuration is a valid kernel instance (Stream asserts it)
  static constexpr bool ok = ok_a16 && ok_chunk && ok_vmcnt && ok_lds && ok_xr;
};

template <int FN_, int MX_, int NW_, int CK_, int D_, bool W4_, bool A16_ = false,
          int XR_ = 0>
struct Stream : StreamGeom<FN_, MX_, NW_, CK_, D_, W4_, A16_, XR_> {
  using G = StreamGeom<FN_, MX_, NW_, CK_, D_, W4_, A16_, XR_>;
  static_assert(G::ok_a16, "A16 takes INT8 weights");
  static_assert(G::ok_chunk, "chunk");
  static_assert(G::ok_vmcnt, "vmcnt range");
  static_assert(G::ok_lds, "LDS");
  static_assert(G::ok_xr, "resident activations: INT8, at most 16 tokens");
};

// Weight copy q (of IW per chunk) of chunk c of the row block starting at
// n0: rows past N re-read the last row, bytes past the row end re-read its
// last 16 (both masked in the MMA).
template <class C>
ZQ_HD inline CopyAddr stream_w_copy(int q, int lane, int n0, int c, int N,
                                    int ldw) {
  const int o = q * 1024 + lane * 16;
  const int row = o / C::CK;
  const int col = ((o % C::CK) >> 4) ^ (row & C::WSW);
  int n = n0 + row;
  n = n < N ? n : N - 1;
  int kb = c * C::CK + col * 16;
  kb = kb < ldw ? kb : ldw - 16;
  return CopyAddr{(int64_t)n * ldw + kb, q * 1024};
}

// The same copy from weights in the chunk-contiguous layout
// [row block][chunk][BN rows][CK bytes] (N % BN == 0, ldw % CK == 0): the
// BN x CK bytes of a chunk are one contiguous range, so the 1024 / CK rows
// of one copy instruction are 1 KB of consecutive bytes (their 16-byte
// columns permuted by the same swizzle).  The LDS image is the row-major
// layout's.
template <class C>
ZQ_HD inline CopyAddr stream_w_copy_chunked(int q, int lane, int rb, int c,
                                            int ldw) {
  const int o = q * 1024 + lane * 16;
  const int row = o / C::CK;
  const int col = ((o % C::CK) >> 4) ^ (row & C::WSW);
  const int64_t chunk = (int64_t)rb * (ldw / C::CK) + c;
  return CopyAddr{(chunk * C::BN + row) * C::CK + col * 16, q * 1024};
}

// Activation copy q (of IXC per chunk) of chunk c: token rows past MX (the
// padding of the last copy) and past M re-read a valid row.  The LDS offset
// is that of the ring slot; a resident chunk image (XR > 0) places the same
// bytes at lds - XOFF from its own base.
template <class C>
ZQ_HD inline CopyAddr stream_x_copy(int q, int lane, int c, int M, int xrow) {
  const int o = q * 1024 + lane * 16;
  int row = o / C::XCK;
  row = row < C::MX ? row : C::MX - 1;       // padding lanes: duplicates
  const int col = ((o % C::XCK) >> 4) ^ (row & C::XSW);
  const int t = row < M ? row : M - 1;
  int kb = c * C::XCK + col * 16;
  kb = kb < xrow ? kb : xrow - 16;
  return CopyAddr{(int64_t)t * xrow + kb, C::XOFF + q * 1024};
}

// Aux dword e of a chunk of the row block at n0: token scales (MX), group
// scales of the block's BN rows, bias dwords (pairs of columns; N is even
// for the rings).
template <class C>
ZQ_HD inline AuxElem stream_aux_elem(int e, int n0, int M, int N, int G) {
  if (e < C::MX) return AuxElem{kAuxSx, e < M ? e : M - 1};
  if (e < C::MX + C::BN) {
    int n = n0 + e - C::MX;
    n = n < N ? n : N - 1;
    return AuxElem{kAuxSw, n / G};
  }
  if (e < C::NAUX) {
    int d = n0 / 2 + (e - C::MX - C::BN);
    const int last = N / 2 - 1;
    return AuxElem{kAuxBias, d < last ? d : last};
  }
  return AuxElem{kAuxPad, 0};
}

}  // namespace zq
