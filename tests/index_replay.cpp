// Host replay of the GEMM kernels' global -> LDS copy addresses (test
// infrastructure; built with the host compiler under AddressSanitizer and
// UBSan by tests/test_index_replay.py).  For every tile and ring
// configuration the kernels instantiate (the generated index_configs.h) and
// every problem shape given on stdin ("M N K bits" per line), it replays
// each copy of each stage of each tile / row block with the same address
// functions the kernels call (zq_index.h) and checks:
//   * the 16 bytes every lane copies lie inside the operand buffer (and are
//     16-byte aligned), and the LDS destination inside its stage region;
//   * every 16-byte chunk of the operands that a fragment read expects
//     (rows inside the tile and inside M / N, k inside K) is present in the
//     LDS stage image, in the swizzled slot that the fragment reads use;
//   * the epilogue-operand gathers (ring and persistent aux dwords) index
//     inside sx [M], sw [N / G] and the bias dwords [N / 2];
//   * the tiled and persistent kernels' workgroup -> tile maps cover every
//     tile exactly once.
// Prints one line per (kernel, configuration) with the copies checked and
// exits non-zero on the first violation.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#define ZQ_HD
#include "zq_index.h"

using namespace zq;

struct Shape {
  int M, N, K, bits;
};

static long long g_checked = 0;

// The clamps act at the edges: replay the first two, the middle and the last
// two indices of each dimension (every index when there are at most five).
static std::vector<int> sample(int n) {
  std::vector<int> v;
  for (int i : {0, 1, n / 2, n - 2, n - 1})
    if (i >= 0 && i < n && (v.empty() || v.back() < i)) v.push_back(i);
  return v;
}

#define REQUIRE(cond, ...)                                     \
  do {                                                         \
    if (!(cond)) {                                             \
      fprintf(stderr, "VIOLATION %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                            \
      fprintf(stderr, "\n");                                   \
      exit(1);                                                 \
    }                                                          \
  } while (0)

// An LDS stage image: for each 16-byte slot, the (row, byte) of the global
// operand copied there (-1: never written).
struct Image {
  std::vector<int64_t> src;
  explicit Image(int bytes) : src(bytes / 16, -1) {}
  void put(int lds, int64_t goff) {
    REQUIRE(lds >= 0 && lds % 16 == 0 && lds / 16 < (int)src.size(),
            "LDS slot %d outside the image", lds);
    src[lds / 16] = goff;
  }
};

template <class C, bool PINGPONG>
static void check_tile(const char *name, const Shape &sh) {
  if (C::W4 != (sh.bits == 4)) return;
  if (C::A16 && sh.bits != 8) return;
  if (sh.K % 64 != 0) return;
  if (PINGPONG && !(sh.N % C::BN == 0 && sh.K % C::KPS == 0 &&
                    sh.K / C::KPS >= C::S))
    return;
  const int ldw = C::W4 ? sh.K / 2 : sh.K;
  const int xb = C::A16 ? 2 : 1;
  const int64_t wbytes = (int64_t)sh.N * ldw, xbytes = (int64_t)sh.M * sh.K * xb;
  const int tiles_n = (sh.N + C::BN - 1) / C::BN;
  const int tiles_m = (sh.M + C::BM - 1) / C::BM;
  const int KT = (sh.K + C::KPS - 1) / C::KPS;
  const bool half_tail = sh.K % C::KPS != 0;
  for (int tn : sample(tiles_n))
    for (int tm : sample(tiles_m))
      for (int kt : sample(KT)) {
        const int n0 = tn * C::BN, m0 = tm * C::BM;
        Image img(C::STAGE);
        for (int q = 0; q < C::IW * C::NWAVES; ++q)
          for (int lane = 0; lane < kWave; ++lane) {
            const CopyAddr a = tile_w_copy<C>(q, lane, n0, kt, sh.N, ldw);
            REQUIRE(a.goff >= 0 && a.goff + 16 <= wbytes && a.goff % 16 == 0,
                    "%s W copy %lld of %lld (M%d N%d K%d tile %d,%d kt %d q %d lane %d)",
                    name, (long long)a.goff, (long long)wbytes, sh.M, sh.N, sh.K,
                    tn, tm, kt, q, lane);
            REQUIRE(a.lds + 1024 <= C::WBYTES, "%s W lds %d", name, a.lds);
            img.put(a.lds + 16 * lane, a.goff);
            ++g_checked;
          }
        for (int q = 0; q < C::IX * C::NWAVES; ++q)
          for (int lane = 0; lane < kWave; ++lane) {
            const CopyAddr a = tile_x_copy<C>(q, lane, m0, kt, sh.M, sh.K);
            REQUIRE(a.goff >= 0 && a.goff + 16 <= xbytes && a.goff % 16 == 0,
                    "%s X copy %lld of %lld (M%d N%d K%d tile %d,%d kt %d q %d lane %d)",
                    name, (long long)a.goff, (long long)xbytes, sh.M, sh.N, sh.K,
                    tn, tm, kt, q, lane);
            REQUIRE(a.lds >= C::WBYTES && a.lds + 1024 <= C::STAGE, "%s X lds %d",
                    name, a.lds);
            img.put(a.lds + 16 * lane, a.goff);
            ++g_checked;
          }
        // every chunk the fragment reads take (swizzled slot of chunk c of
        // row r) holds that chunk of the operand; the unused upper half of
        // a half stage is not read
        const int wlim = (kt == KT - 1 && half_tail) ? C::WROW / 2 : C::WROW;
        for (int r = 0; r < C::BN && n0 + r < sh.N; ++r)
          for (int c = 0; c * 16 < wlim; ++c) {
            const int slot = r * C::WCPR + wswz<C::WROW>(c, r);
            const int64_t want = (int64_t)(n0 + r) * ldw + kt * C::WROW + 16 * c;
            REQUIRE(img.src[slot] == want, "%s W image row %d chunk %d kt %d: %lld != %lld",
                    name, r, c, kt, (long long)img.src[slot], (long long)want);
          }
        const int xlim = (kt == KT - 1 && half_tail) ? C::XROW / 2 : C::XROW;
        for (int r = 0; r < C::BM && m0 + r < sh.M; ++r)
          for (int c = 0; c * 16 < xlim; ++c) {
            const int slot = C::WBYTES / 16 + r * C::XCPR + wswz<C::XROW>(c, r);
            const int64_t want = (int64_t)(m0 + r) * sh.K * xb + kt * C::XROW + 16 * c;
            REQUIRE(img.src[slot] == want, "%s X image row %d chunk %d kt %d", name, r,
                    c, kt);
          }
      }
  if (!PINGPONG) {
    // the tiled kernel's workgroup -> tile map: every tile exactly once
    const int total = tiles_m * tiles_n;
    std::vector<int> seen(total, 0);
    for (int b = 0; b < total; ++b) {
      int tm, tn;
      grouped_tile<kTileGroup>(xcd_remap(b, total), tiles_m, tiles_n, tm, tn);
      REQUIRE(tm >= 0 && tm < tiles_m && tn >= 0 && tn < tiles_n, "%s tile", name);
      ++seen[tn * tiles_m + tm];
    }
    for (int i = 0; i < total; ++i)
      REQUIRE(seen[i] == 1, "%s tile %d run %d times", name, i, seen[i]);
  }
  if (PINGPONG) {
    // the persistent aux gathers and the logical tile map (every tile once)
    for (int G : {32, 64, 128}) {
      if (sh.N % G) continue;
      for (int tn : sample(tiles_n))
        for (int tm : sample(tiles_m))
          for (int e = 0; e < PAux<C>::NCOPY * 64; ++e) {
            const AuxElem a = persist_aux_elem<C>(e, tn * C::BN, tm * C::BM, sh.M, G);
            if (a.src == kAuxBias)
              REQUIRE(a.index >= 0 && 2 * a.index + 1 < sh.N, "%s bias dword %d", name,
                      a.index);
            if (a.src == kAuxSx) REQUIRE(a.index >= 0 && a.index < sh.M, "%s sx", name);
            if (a.src == kAuxSw)
              REQUIRE(a.index >= 0 && a.index < sh.N / G, "%s sw %d", name, a.index);
            ++g_checked;
          }
    }
    const int total = tiles_m * tiles_n, grid = total < 256 ? total : 256;
    std::vector<int> seen(total, 0);
    for (int b = 0; b < grid; ++b) {
      const int slot = xcd_remap(b, grid);
      for (int L = slot; L < total; L += grid) {
        int tm, tn;
        persist_tile(L, tiles_m, tiles_n, tm, tn);
        REQUIRE(tm >= 0 && tm < tiles_m && tn >= 0 && tn < tiles_n, "%s tile", name);
        ++seen[tn * tiles_m + tm];
      }
    }
    for (int i = 0; i < total; ++i) REQUIRE(seen[i] == 1, "%s tile %d run %d times", name, i, seen[i]);
  }
}

template <class C>
static void check_stream(const char *name, const Shape &sh) {
  if (C::W4 != (sh.bits == 4)) return;
  if (C::A16 && sh.bits != 8) return;
  if (sh.M > C::MX || (sh.N & 1) || sh.K % 64) return;
  const int ldw = C::W4 ? sh.K / 2 : sh.K;
  const int xrow = C::A16 ? 2 * sh.K : sh.K;
  const int64_t wbytes = (int64_t)sh.N * ldw, xbytes = (int64_t)sh.M * xrow;
  const int NRB = (sh.N + C::BN - 1) / C::BN;
  const int NC = (ldw + C::CK - 1) / C::CK;
  // resident activations: launched only when a wave's chunks fit
  if (C::XR > 0 && (NC + C::NW - 1) / C::NW > C::XR) return;
  for (int rb : sample(NRB))
    for (int c : sample(NC)) {
      const int n0 = rb * C::BN;
      Image img(C::SLOT);
      for (int q = 0; q < C::IW; ++q)
        for (int lane = 0; lane < kWave; ++lane) {
          const CopyAddr a = stream_w_copy<C>(q, lane, n0, c, sh.N, ldw);
          REQUIRE(a.goff >= 0 && a.goff + 16 <= wbytes && a.goff % 16 == 0,
                  "%s W copy %lld of %lld (M%d N%d K%d rb %d c %d)", name,
                  (long long)a.goff, (long long)wbytes, sh.M, sh.N, sh.K, rb, c);
          REQUIRE(a.lds + 1024 <= C::XOFF, "%s W lds", name);
          img.put(a.lds + 16 * lane, a.goff);
          ++g_checked;
        }
      // activations: in the ring slot (XR == 0), or in the chunk's
      // resident image, copied once per launch (XR > 0), whose slots are
      // checked here shifted by XOFF so that one image serves both
      Image ximg(C::XOFF + C::XCH);
      for (int q = 0; q < C::IXC; ++q)
        for (int lane = 0; lane < kWave; ++lane) {
          const CopyAddr a = stream_x_copy<C>(q, lane, c, sh.M, xrow);
          REQUIRE(a.goff >= 0 && a.goff + 16 <= xbytes && a.goff % 16 == 0,
                  "%s X copy %lld of %lld (M%d N%d K%d c %d)", name,
                  (long long)a.goff, (long long)xbytes, sh.M, sh.N, sh.K, c);
          if (C::XR == 0) {
            REQUIRE(a.lds >= C::XOFF && a.lds + 1024 <= C::AOFF, "%s X lds", name);
          } else {
            REQUIRE(a.lds >= C::XOFF && a.lds - C::XOFF + 1024 <= C::XCH,
                    "%s resident X lds", name);
          }
          ximg.put(a.lds + 16 * lane, a.goff);
          ++g_checked;
        }

      // chunks read: weight row r, 16-byte column j of the chunk (inside
      // the row), activation row t < M, column j of its XCK bytes
      for (int r = 0; r < C::BN && n0 + r < sh.N; ++r)
        for (int j = 0; j < C::CK / 16 && c * C::CK + 16 * j < ldw; ++j) {
          const int slot = (r * C::CK) / 16 + (j ^ (r & C::WSW));
          const int64_t want = (int64_t)(n0 + r) * ldw + c * C::CK + 16 * j;
          REQUIRE(img.src[slot] == want, "%s W image r %d j %d c %d", name, r, j, c);
        }
      // the chunk-contiguous weight layout (where the shape tiles into it):
      // the same LDS image from one contiguous range per chunk, and every
      // copy instruction reads 1 KB of consecutive bytes
      if (sh.N % C::BN == 0 && ldw % C::CK == 0) {
        Image cimg(C::SLOT);
        for (int q = 0; q < C::IW; ++q) {
          int64_t lo = INT64_MAX, hi = -1;
          for (int lane = 0; lane < kWave; ++lane) {
            const CopyAddr a = stream_w_copy_chunked<C>(q, lane, rb, c, ldw);
            REQUIRE(a.goff >= 0 && a.goff + 16 <= wbytes && a.goff % 16 == 0,
                    "%s chunked W copy %lld of %lld (N%d K%d rb %d c %d)",
                    name, (long long)a.goff, (long long)wbytes, sh.N, sh.K,
                    rb, c);
            REQUIRE(a.lds == q * 1024, "%s chunked W lds", name);
            cimg.put(a.lds + 16 * lane, a.goff);
            lo = a.goff < lo ? a.goff : lo;
            hi = a.goff > hi ? a.goff : hi;
            ++g_checked;
          }
          REQUIRE(hi - lo == 1024 - 16 && lo % 1024 == 0,
                  "%s chunked copy %d not one 1 KB run", name, q);
        }
        for (int r = 0; r < C::BN; ++r)
          for (int j = 0; j < C::CK / 16; ++j) {
            const int slot = (r * C::CK) / 16 + (j ^ (r & C::WSW));
            const int64_t want =
                (((int64_t)rb * (ldw / C::CK) + c) * C::BN + r) * C::CK + 16 * j;
            REQUIRE(cimg.src[slot] == want, "%s chunked W image r %d j %d c %d",
                    name, r, j, c);
          }
      }
      for (int t = 0; t < sh.M; ++t)
        for (int j = 0; j < C::XCK / 16 && c * C::XCK + 16 * j < xrow; ++j) {
          const int slot = C::XOFF / 16 + (t * C::XCK) / 16 + (j ^ (t & C::XSW));
          const int64_t want = (int64_t)t * xrow + c * C::XCK + 16 * j;
          REQUIRE(ximg.src[slot] == want, "%s X image t %d j %d c %d", name, t, j, c);
        }
      for (int G : {1, 2, 32, 64, 128}) {
        if (sh.N % G) continue;
        for (int e = 0; e < C::IA * 64; ++e) {
          const AuxElem a = stream_aux_elem<C>(e, n0, sh.M, sh.N, G);
          if (a.src == kAuxBias)
            REQUIRE(a.index >= 0 && 2 * a.index + 1 < sh.N, "%s bias dword", name);
          if (a.src == kAuxSx) REQUIRE(a.index >= 0 && a.index < sh.M, "%s sx", name);
          if (a.src == kAuxSw) REQUIRE(a.index >= 0 && a.index < sh.N / G, "%s sw", name);
          ++g_checked;
        }
      }
    }
}

// A configuration is replayed only where it is a valid kernel instance (the
// generated list expands the W4 parameter both ways).
template <bool PP, int BN, int BM, int WN, int WM, int S, bool W4, int KB = 128,
          bool A16 = false>
static void try_tile(const char *name, const Shape &sh) {
  if constexpr (TileGeom<BN, BM, WN, WM, S, W4, KB, A16>::ok)
    check_tile<Tile<BN, BM, WN, WM, S, W4, KB, A16>, PP>(name, sh);
}

template <int FN, int MX, int NW, int CK, int D, bool W4, bool A16 = false,
          int XR = 0>
static void try_stream(const char *name, const Shape &sh) {
  if constexpr (StreamGeom<FN, MX, NW, CK, D, W4, A16, XR>::ok)
    check_stream<Stream<FN, MX, NW, CK, D, W4, A16, XR>>(name, sh);
}

#include "index_configs.h"

int main() {
  std::vector<Shape> shapes;
  Shape s;
  while (scanf("%d %d %d %d", &s.M, &s.N, &s.K, &s.bits) == 4) shapes.push_back(s);
  for (const Shape &sh : shapes) {
    const long long before = g_checked;
#define ZQ_TILE(...) try_tile<false, __VA_ARGS__>("tile<" #__VA_ARGS__ ">", sh);
#define ZQ_PINGPONG(...) try_tile<true, __VA_ARGS__>("pingpong<" #__VA_ARGS__ ">", sh);
#define ZQ_STREAM(...) try_stream<__VA_ARGS__>("stream<" #__VA_ARGS__ ">", sh);
    ZQ_CONFIGS
    printf("M=%d N=%d K=%d W%d: %lld addresses\n", sh.M, sh.N, sh.K, sh.bits,
           g_checked - before);
  }
  printf("OK %zu shapes, %lld addresses checked\n", shapes.size(), g_checked);
  return 0;
}
