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
#ifndef HYB_GEMM_SPLIT_COST
#define HYB_GEMM_SPLIT_COST 30.0
#endif
#ifndef HYB_GEMM_LDS_SPLIT_ROUND
#define HYB_GEMM_LDS_SPLIT_ROUND 0.39
#endif
// K parts of the 192- and 256-token LDS tiles: the fewest K steps a part
// walks; and, for parts that follow whole rounds of a plain launch, a fixed
// time (us) plus a time per parts workgroup (its 256 KiB partial tile
// written and read back, about 0.08 us at 6.7 TB/s)
#ifndef HYB_GEMM_PART_MIN_STEPS
#define HYB_GEMM_PART_MIN_STEPS 16
#endif
#ifndef HYB_GEMM_TAIL_FIXED_US
#define HYB_GEMM_TAIL_FIXED_US 10.0
#endif
#ifndef HYB_GEMM_TAIL_WG_US
#define HYB_GEMM_TAIL_WG_US 0.078
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

// Whole slabs of the mixed decode launch.  Workgroup b runs on XCD b % 8
// and the CUs of an XCD take its workgroups in turn, so with S slabs on C
// CUs the last round leaves r = S mod C CUs a slab more than the rest, and
// the launch waits on them.  Where 2r <= C those r slabs are cut into 8-row
// halves, one per CU of the last round, and the other slabs stay whole.
int64_t gemv_full_slabs(int64_t slabs, int cus) {
  const int64_t r = cus > 0 ? slabs % cus : 0;
  return (slabs > cus && r > 0 && 2 * r <= cus) ? slabs - r : slabs;
}

bool gemv_preferred(const hyb_layout& L, int m) {
  if (m <= kGemvCrossoverM) return true;
  // 5-16 tokens on a matrix of at most one 16-row slab per CU: the decode
  // kernel's 8 or 16 wavefronts per slab match or beat the matrix-core
  // product there (1024-4096 rows: K = 8192-28672 1.0-1.5x faster, K = 4096
  // within 8%).  With more slabs the matrix cores win: at 5-8 tokens 14336 x
  // 4096, 6144 x 4096 and 5120 x 17408 take 16.7, 11.7 and 37-39 us against
  // 22, 16 and 41-42 us (8192 x 28672 even); at 9-16 tokens 5120 x 17408 and
  // 6144 x 4096 take 41-45 and 12-13 us against 64-69 and 22 us.
  return m <= kMaxGemvM && L.n / 16 <= int64_t(device_cus());
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
//
// A register-fed shape whose last round of workgroups would leave compute
// units idle can instead split K over one workgroup per CU (the stream-K
// schedule of k_gemm_split), which then takes tiles / CUs of a round plus a
// fixed cost of kSplitCost / S rounds for S K steps per tile (the partial
// sums, the pieces' pipeline starts and the second kernel that adds them).
// Measured on 1024 to 28672 rows, K = 4096 to 28672, 16 to 300 tokens: a
// cost of 30 K steps picks the faster of plain and split in every case but
// one (28672 x 8192 at 128 tokens, where the LDS shape runs, 7% slower).
namespace {

constexpr double kSplitCost = HYB_GEMM_SPLIT_COST;
// Cost of one round of the split LDS-fed 64-token shape on the scale of
// kRound (register-fed 64 tokens x 128 rows: 0.29), for S K steps per tile.
// Against the split register-fed shapes it grows with K: measured 0.37-0.44
// at 64-80 K steps, 0.44-0.49 at 128, 0.46-0.56 at 224-448.
double lds_split_round(int64_t steps) {
  const double c = HYB_GEMM_LDS_SPLIT_ROUND + 0.0007 * double(steps - 64);
  return c < HYB_GEMM_LDS_SPLIT_ROUND ? HYB_GEMM_LDS_SPLIT_ROUND : (c > 0.6 ? 0.6 : c);
}
// The same for the split LDS-fed 128-token shape.  Up to 128 tokens it is
// priced against the split register-fed shapes (0.47: 8192 x 28672 at 128
// tokens 103 us against 119, 28672 x 8192 at 128 112 against 124 for the
// LDS 64-token round); above 128 against the LDS rounds, growing with K
// (0.63 at 64 K steps to 0.78 at 448: 17408 x 5120 at 256 tokens 79 us
// against 93 for the 128-token round, 8192 x 28672 at 256 and 512 tokens
// 167 and 291 us against 187 and 367).
double lds8_split_round(int64_t steps, bool up_to_128) {
  if (up_to_128) return 0.47;
  const double c = 0.63 + 0.0004 * double(steps - 64);
  return c < 0.63 ? 0.63 : (c > 0.8 ? 0.8 : c);
}

struct Priced {
  GemmRoute r;
  double rounds;  // rounds of this shape's workgroups over the CUs
};

// The cheaper of the plain and the split launch of one register-fed shape
// (steps: K steps of 64 columns per tile).  A plain launch costs its
// workgroups per CU, rounded up; with two workgroups per CU resident (the
// shapes of rx_occupancy) the second still shares the CU, which costs about
// as much as running after the first.
Priced rx_priced(int64_t n, int64_t steps, int64_t m, int mb, int waves, int rg, int64_t cus) {
  const int64_t gn = (n + 64 * rg - 1) / (64 * rg), gm = (m + 16 * mb - 1) / (16 * mb);
  const int64_t tiles = gn * gm;
  const int64_t rounds = (tiles + cus - 1) / cus;
  Priced p{GemmRoute{kRouteRegister, mb, waves, rg, 0}, double(rounds)};
  // Each wavefront of a split workgroup keeps at least kSplitMinSteps K
  // steps; every token block gets the same number of workgroups.
  int64_t groups = tiles * steps / (int64_t(waves) * kSplitMinSteps);
  const int64_t max_groups = cus < kSplitMaxCus ? cus : kSplitMaxCus;
  if (groups > max_groups) groups = max_groups;
  groups -= groups % gm;
  if (tiles % cus != 0 && groups > 1 && gn * steps < (int64_t(1) << 31)) {
    const double c = double(tiles) / double(groups) + kSplitCost / double(steps);
    if (c < p.rounds) p = Priced{GemmRoute{kRouteSplit, mb, waves, rg, int32_t(groups)}, c};
  }
  return p;
}

}  // namespace

size_t split_workspace_bytes(const GemmRoute& r) {
  if (r.kernel != kRouteSplit) return 0;
  // two partial tiles per workgroup of a stream-K range; one per workgroup
  // of the 192- and 256-token LDS tiles, whose K is cut into equal parts
  const size_t pieces = (r.rg == 4 && r.mb >= 12) ? 1 : 2;
  return size_t(r.groups) * pieces * size_t(r.rg) * size_t(r.mb) * 4096;
}

GemmRoute gemm_route(int64_t n, int64_t k, int m, int64_t cus) {
  const int64_t groups = n / 64;  // 64-row workgroups of the register-fed kernel
  const int64_t steps = (k + 63) / 64;
  const int64_t m64 = m;  // token-block counts in int64: m may be close to INT32_MAX
  if (m <= 16) {
    // Eight wavefronts (one workgroup per CU) when the 64-row groups fit in
    // one round, else four (two workgroups per CU); split as priced above.
    return rx_priced(n, steps, m64, 1, groups <= cus ? 8 : 4, 1, cus).r;
  }
  // Register-fed shapes: token blocks of 16 per workgroup, wavefronts, 64-row
  // groups per workgroup; and the time of one round of each, relative to one
  // round of the 256-token LDS shape over the same K (measured on 1024 to
  // 8192 rows, K = 4096 to 28672, 24 to 1024 tokens).
  // (32 tokens x 128 rows on four wavefronts runs ahead of 64 tokens x 64
  // rows on eight: of equal rounds it was the faster in every case measured.)
  // (48 tokens x 128 rows costs less per round than 64 x 128: it needs
  // fewer registers; 0.26 against 0.29 on 8192 and 17408 rows, and split
  // 0.23, where the 64-token shape's split kernel spills.)
  constexpr int kNumShapes = 6;
  constexpr int kShapes[kNumShapes][3] = {{1, 8, 1}, {2, 8, 1}, {2, 4, 2}, {4, 8, 1}, {3, 4, 2}, {4, 4, 2}};
  constexpr double kRound[kNumShapes] = {0.12, 0.155, 0.21, 0.21, 0.26, HYB_GEMM_C_RX};
  constexpr double kSplitRound[kNumShapes] = {0.12, 0.155, 0.21, 0.21, 0.23, HYB_GEMM_C_RX};
  auto rx_wgs = [&](int i) {
    return ((groups + kShapes[i][2] - 1) / kShapes[i][2]) * ((m64 + 16 * kShapes[i][0] - 1) / (16 * kShapes[i][0]));
  };
  // The cheapest split launch of any register-fed shape (cost relative to
  // the 256-token LDS round, as kRound).
  auto best_split = [&](double& cost, bool up_to_128) {
    GemmRoute best{0, 0, 0, 0, 0};
    for (int i = 0; i < kNumShapes; ++i) {
      if ((m64 + 16 * kShapes[i][0] - 1) / (16 * kShapes[i][0]) > 65535) continue;
      const Priced p = rx_priced(n, steps, m64, kShapes[i][0], kShapes[i][1], kShapes[i][2], cus);
      if (p.r.kernel == kRouteSplit && (best.kernel == 0 || p.rounds * kSplitRound[i] < cost)) {
        best = p.r;
        cost = p.rounds * kSplitRound[i];
      }
    }
    // Up to 128 tokens, the LDS-fed 64-token shape (256 rows on eight
    // wavefronts) split the same way: per unit of work it is the cheaper
    // kernel where its tiles fill the CUs (65536 x 4096 at 64 tokens: one
    // round of it 83 us, against 105 us for two rounds of 64 tokens x 128
    // rows; 17408 x 5120 at 64 and 128 tokens: 37 and 53 us against 41 and
    // 57 us for the split register-fed shape).  Above 128 tokens it lost to
    // the shapes priced here in every case measured (8192 x 28672 and 4096 x
    // 14336 at 256 tokens by 9-10%, 14336 x 4096 at 256 by 13%).
    const Priced lp = rx_priced(n, steps, m64, 4, 8, 4, cus);
    if (up_to_128 && lp.r.kernel == kRouteSplit && (best.kernel == 0 || lp.rounds * lds_split_round(steps) < cost)) {
      best = lp.r;
      cost = lp.rounds * lds_split_round(steps);
    }
    // From 97 tokens (a 128-token block at least 3/4 full), the LDS-fed
    // 128-token shape split the same way: per K step it does twice the
    // 64-token shape's products for 1.3x its loads.
    if (m64 > 96) {
      const Priced lp8 = rx_priced(n, steps, m64, 8, 8, 4, cus);
      const double c8 = lp8.rounds * lds8_split_round(steps, up_to_128);
      if (lp8.r.kernel == kRouteSplit && (best.kernel == 0 || c8 < cost)) {
        best = lp8.r;
        cost = c8;
      }
    }
    // Above 128 tokens, the 192- and 256-token LDS tiles with K cut into
    // equal parts (k_gemm_lds_parts), when their tiles fill at most half the
    // CUs.  Priced by time: each workgroup walks S / parts K steps at 1.45 or
    // 1.75 us a step (measured at full occupancy), plus a fixed 25 us and
    // 0.05 us per K step of the tile (the sum kernel, the pieces' pipeline
    // starts); one round of the 256-token LDS tile costs about 1.75 us per K
    // step, which converts the time to this scale.
    //
    // With more tiles than CUs, the 256-token tiles can end a launch instead:
    // the row blocks whose tiles fill whole rounds of the CUs run in one
    // plain launch (a round costs 1), and the blocks after them, which would
    // leave most CUs idle in a last round, run with K cut into parts over
    // the CUs.  Measured against the previous route (graph bursts, 25
    // products of 4096-28672 rows at 1024-4096 tokens): 17408 x 5120 at
    // 1024 / 2048 / 3072 / 4096 tokens 255 / 367 / 546 / 691 us -> 212 /
    // 343 / 486 / 623; 28672 x 8192 at 2048 and 3072 884 and 1307 -> 837 and
    // 1275; 14336 x 4096 at 4096 432 -> 426.  The same with the 192-token
    // tile lost more often than it won (28672 x 8192 at 1536 tokens 3% slower,
    // 14336 x 4096 and 8192 x 28672 at 2048 10-20% slower), so it is not
    // offered.
    if (!up_to_128) {
      for (const int mb : {12, 16}) {
        const int64_t gn = (n + 255) / 256, gm = (m64 + 16 * mb - 1) / (16 * mb), tiles = gn * gm;
        const double step_us = mb == 12 ? 1.45 : 1.75;
        int64_t parts = cus / tiles;
        if (parts > steps / HYB_GEMM_PART_MIN_STEPS) parts = steps / HYB_GEMM_PART_MIN_STEPS;
        if (parts >= 2 && tiles * parts <= kSplitMaxCus) {
          const double t_us = step_us * double(steps) / double(parts) + 25.0 + 0.05 * double(steps);
          const double c = t_us / (1.75 * double(steps));
          if (best.kernel == 0 || c < cost) {
            best = GemmRoute{kRouteSplit, mb, 8, 4, int32_t(tiles * parts), 0};
            cost = c;
          }
          continue;
        }
        if (mb != 16) continue;
        const int64_t rows0 = (tiles / cus) * cus / gm;  // whole row blocks in whole rounds
        if (rows0 < 1 || rows0 >= gn) continue;
        const int64_t tail = (gn - rows0) * gm;
        int64_t tparts = cus / tail;
        if (tparts > steps / HYB_GEMM_PART_MIN_STEPS) tparts = steps / HYB_GEMM_PART_MIN_STEPS;
        if (tparts < 2 || tail * tparts > kSplitMaxCus) continue;
        const double t_us = step_us * double(steps) / double(tparts) + HYB_GEMM_TAIL_FIXED_US +
                            HYB_GEMM_TAIL_WG_US * double(tail * tparts) + 0.05 * double(steps);
        const double c = double((rows0 * gm + cus - 1) / cus) + t_us / (1.75 * double(steps));
        if (best.kernel == 0 || c < cost) {
          best = GemmRoute{kRouteSplit, mb, 8, 4, int32_t(tail * tparts), int32_t(rows0)};
          cost = c;
        }
      }
    }
    return best;
  };
  auto rx = [&](int i) { return GemmRoute{kRouteRegister, kShapes[i][0], kShapes[i][1], kShapes[i][2], 0}; };
  if (m <= 128) {
    // The fewest rounds of workgroups over the CUs wins, then the most
    // workgroups; on a tie the earlier entry (one row group before two,
    // then the smaller token block).  Measured on 1024 to 17408 rows at
    // 17-128 tokens: the pick is the fastest shape or within 3% of it.
    int best = 0;
    int64_t best_rounds = 0, best_wgs = 0;
    for (int i = 0; i < kNumShapes; ++i) {
      const int64_t wgs = rx_wgs(i);
      const int64_t rounds = (wgs + cus - 1) / cus;
      if (i == 0 || rounds < best_rounds || (rounds == best_rounds && wgs > best_wgs)) {
        best = i;
        best_rounds = rounds;
        best_wgs = wgs;
      }
    }
    double plain = double(best_rounds) * kRound[best];
    GemmRoute pick = rx(best);
    // A wide matrix can need two rounds of the 128-row x 64-token shape
    // while the 64-token LDS shape (256 rows per workgroup) fits the whole
    // product in one; that round is cheaper than two (28672 x 8192 at 80-128
    // tokens: 125 against 145-160 us; 17408 x 5120 at 128: 73 against 77).
    if (best == kNumShapes - 1 && best_rounds >= 2 && ((n + 255) / 256) * ((m64 + 63) / 64) <= cus) {
      pick = GemmRoute{kRouteLds, 4, 8, 4, 0};
      plain = 0.57;
    }
    double split = 0.0;
    const GemmRoute s = best_split(split, true);
    return (s.kernel == kRouteSplit && split < plain) ? s : pick;
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
  for (int i = 0; i < kNumShapes; ++i) {
    if ((m64 + 16 * kShapes[i][0] - 1) / (16 * kShapes[i][0]) > 65535) continue;
    const double c = double((rx_wgs(i) + cus - 1) / cus) * kRound[i];
    if (rx_best < 0 || c < rx_cost) {
      rx_best = i;
      rx_cost = c;
    }
  }
  double split = 0.0;
  const GemmRoute s = best_split(split, false);
  if (s.kernel == kRouteSplit && split < rx_cost && split < best) return s;
  if (rx_best >= 0 && rx_cost < 0.9 * best) return rx(rx_best);
  if (c256 == best) return GemmRoute{kRouteLds, 16, 8, 4, 0};
  if (c192 == best) return GemmRoute{kRouteLds, 12, 8, 4, 0};
  if (c128 == best) return GemmRoute{kRouteLds, 8, 8, 4, 0};
  return GemmRoute{kRouteLds, 4, 8, 4, 0};
}

GemmRoute gemm_route(const hyb_layout& L, int m, int64_t cus) { return gemm_route(L.n, L.tiles_k * L.b2, m, cus); }

GemmRoute gemm_route_device(const hyb_layout& L, int m) {
  if (gemv_preferred(L, m)) return GemmRoute{kRouteDecode, 0, gemv_waves(L.n / 16, m), 0, 0};
  return gemm_route(L, m, device_cus());
}

}  // namespace hyb
