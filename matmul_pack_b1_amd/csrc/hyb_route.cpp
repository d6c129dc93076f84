// Host-only routing of libhyb: which kernel and launch shape a product
// runs for a given matrix, token count and compute-unit count.  Pure host
// arithmetic (no kernels), kept apart from the kernel files so that it can
// be built by the host compiler alone.
#include <atomic>
#include <cstdint>

#include "hyb_internal.h"

#ifndef HYB_GEMM_C192
#define HYB_GEMM_C192 0.8
#endif
#ifndef HYB_GEMM_C_RX
#define HYB_GEMM_C_RX 0.29
#endif

namespace hyb {

// Compute units of the current device (cached per device; callers on
// several host threads may race to fill an entry with the same value).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Wavefronts per slab of the decode kernels.  Four when the slabs fill the
// CUs at least twice (each wavefront walks a quarter of the tile row); a
// shorter matrix has too few workgroups to keep enough loads in flight, so
// its tile row is split eight ways (up to 4 tokens) or sixteen (more
// tokens).  Measured on 1024 and 4096 rows: 1.2x at 1 token, 1.2-1.3x at 4,
// 1.8-1.9x at 16; on 14336 rows four stay best.
int gemv_waves(int64_t slabs, int m) {
  if (slabs >= 2 * int64_t(device_cus())) return kGemvWaves;
  return m <= 4 ? 8 : 16;
}

bool gemv_preferred(const hyb_layout& L, int m) {
  if (m <= kGemvCrossoverM) return true;
  // 9-16 tokens on a matrix short enough for 16 wavefronts per slab: the
  // decode kernel beats the register-fed product there (1024 and 4096 rows
  // at 16 tokens: 11-12 us against 15-16 us)
  return m <= kMaxGemvM && gemv_waves(L.n / 16, m) == 16;
}

// Workgroup shape by token count.  Up to 16 tokens the register-fed kernel
// k_gemm_rx runs 16 tokens x 64 rows per workgroup.  Up to 128 tokens it
// runs in the shape that fills the CUs best (one exception below for wide
// matrices at 65-128 tokens).  From 129 tokens one of four LDS-fed shapes
// runs, 256 weight rows by BM = 256, 192, 128 or 64 tokens.  Every
// workgroup walks all of K, so the time is the number of rounds of
// workgroups over the compute units times the time of one workgroup; the
// relative step costs of the shapes are measured (a 256-token step costs 1,
// a 192-token step 0.8, a 128-token step 0.64, a 64-token step 0.57), and
// the shape with the smallest product runs, unless a register-fed shape,
// priced the same way, costs under 0.9 of it.
GemmRoute gemm_route(int64_t n, int m, int64_t cus) {
  const int64_t groups = n / 64;  // 64-row workgroups of the register-fed kernel
  if (m <= 16) {
    // Eight wavefronts (one workgroup per CU) when the 64-row groups fit in
    // one round, else four (two workgroups per CU).
    return GemmRoute{kRouteRegister, 1, groups <= cus ? 8 : 4, 1};
  }
  // Register-fed shapes: token blocks of 16 per workgroup, wavefronts, 64-row
  // groups per workgroup; and the time of one round of each, relative to one
  // round of the 256-token LDS shape over the same K (measured on 1024 to
  // 8192 rows, K = 4096 to 28672, 24 to 1024 tokens).
  constexpr int kShapes[5][3] = {{1, 8, 1}, {2, 8, 1}, {4, 8, 1}, {2, 4, 2}, {4, 4, 2}};
  constexpr double kRound[5] = {0.12, 0.155, 0.21, 0.21, HYB_GEMM_C_RX};
  // token-block counts in int64: m may be close to INT32_MAX
  const int64_t m64 = m;
  auto rx_wgs = [&](int i) {
    return ((groups + kShapes[i][2] - 1) / kShapes[i][2]) * ((m64 + 16 * kShapes[i][0] - 1) / (16 * kShapes[i][0]));
  };
  auto rx = [&](int i) { return GemmRoute{kRouteRegister, kShapes[i][0], kShapes[i][1], kShapes[i][2]}; };
  if (m <= 128) {
    // The fewest rounds of workgroups over the CUs wins, then the most
    // workgroups; on a tie the earlier entry (one row group before two,
    // then the smaller token block).  Measured on 1024 to 17408 rows at
    // 17-128 tokens: the pick is the fastest shape or within 3% of it.
    int best = 0;
    int64_t best_rounds = 0, best_wgs = 0;
    for (int i = 0; i < 5; ++i) {
      const int64_t wgs = rx_wgs(i);
      const int64_t rounds = (wgs + cus - 1) / cus;
      if (i == 0 || rounds < best_rounds || (rounds == best_rounds && wgs > best_wgs)) {
        best = i;
        best_rounds = rounds;
        best_wgs = wgs;
      }
    }
    // A wide matrix can need two rounds of the 128-row x 64-token shape
    // while the 64-token LDS shape (256 rows per workgroup) fits the whole
    // product in one; that round is cheaper than two (28672 x 8192 at 80-128
    // tokens: 125 against 145-160 us; 17408 x 5120 at 128: 73 against 77).
    if (best == 4 && best_rounds >= 2 && ((n + 255) / 256) * ((m64 + 63) / 64) <= cus)
      return GemmRoute{kRouteLds, 4, 8, 4};
    return rx(best);
  }
  const int64_t gn = (n + 255) / 256;
  auto cost = [&](int64_t bm, double step) {
    return double((gn * ((m + bm - 1) / bm) + cus - 1) / cus) * step;
  };
  const double c256 = cost(256, 1.0), c192 = cost(192, HYB_GEMM_C192), c128 = cost(128, 0.64), c64 = cost(64, 0.57);
  const double best = c256 < c192 ? (c256 < c128 ? (c256 < c64 ? c256 : c64) : (c128 < c64 ? c128 : c64))
                                  : (c192 < c128 ? (c192 < c64 ? c192 : c64) : (c128 < c64 ? c128 : c64));
  // A matrix with few 256-row blocks (a short one, or a short and deep one
  // such as 8192 x 28672) leaves most CUs idle under every LDS shape; the
  // cheapest register-fed shape runs when it costs under 0.9 of the best LDS
  // shape (e.g. 1024 x 4096 at 160-1024 tokens: 1.3-1.9x faster; 8192 x
  // 28672 at 160-256 tokens: 382 -> 169-231 us).  A shape needing more than
  // 65535 token blocks, the register-fed grid's limit, is not a candidate.
  int rx_best = -1;
  double rx_cost = 0.0;
  for (int i = 0; i < 5; ++i) {
    if ((m64 + 16 * kShapes[i][0] - 1) / (16 * kShapes[i][0]) > 65535) continue;
    const double c = double((rx_wgs(i) + cus - 1) / cus) * kRound[i];
    if (rx_best < 0 || c < rx_cost) {
      rx_best = i;
      rx_cost = c;
    }
  }
  if (rx_best >= 0 && rx_cost < 0.9 * best) return rx(rx_best);
  if (c256 == best) return GemmRoute{kRouteLds, 16, 8, 4};
  if (c192 == best) return GemmRoute{kRouteLds, 12, 8, 4};
  if (c128 == best) return GemmRoute{kRouteLds, 8, 8, 4};
  return GemmRoute{kRouteLds, 4, 8, 4};
}

GemmRoute gemm_route_device(const hyb_layout& L, int m) {
  if (gemv_preferred(L, m)) return GemmRoute{kRouteDecode, 0, gemv_waves(L.n / 16, m), 0};
  return gemm_route(L.n, m, device_cus());
}

}  // namespace hyb
