// Decode kernels of libhyb (gfx950): the tile-hybrid GEMV for 1-16 tokens,
// its grouped launch over several matrices sharing x, and its sparse +
// low-rank variant.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hyb_device.h"

namespace hyb {
namespace {

// ---------------------------------------------------------------- GEMV ----
//
// y[m, n] = sum_k W'[n, k] x[m, k] for m < M <= 16.
// One workgroup = one 16-row slab; its WAVES wavefronts split the tile
// columns of the slab's tile row into contiguous ranges.  Per tile a
// wavefront loads the slab piece (dense: b2/32 x 16 B per lane; sparse: b2/64
// x 16 B of values plus b2/64 16-bit metadata words per lane) and this tile's
// x columns (MT x b2), stages x in its own LDS region, and accumulates in
// fp32 with v_dot2.  Sparse 2:4 groups gather their two x values with one
// v_perm each; 4:8 groups are expanded to their eight columns with v_perm
// selectors from a per-workgroup LDS table of all 256 mask bytes.  Loads run one tile ahead through a two-stage register ring (the
// loop is unrolled by two so no in-flight register is ever copied).  Lanes
// L, L^16, L^32, L^48 hold the same row and are combined with cross-lane
// swizzles; the wavefronts are then summed in a fixed order through LDS, so
// results are reproducible run to run.
// x staging of the decode kernel.  Per tile (XR = false) every wavefront
// loads the tile's MT x b2 block of x with its weights and stages it in its
// own LDS region.  With XR = true a wavefront loads the x columns of its whole
// tile range once, before its first weight loads, with full 1 KiB loads
// (4 KiB per token row: up to 2048 / b2 tiles); the per-tile x loads, which
// carried only MT x b2 x 2 bytes each, go away (measured 0.3 us on the 8B up
// projection at one token).
template <int B2>
constexpr int kXrTiles = 2048 / B2;

template <int MT, int B2, bool XR>
struct GemvStage {
  static constexpr int kXPieces = XR ? 0 : MT * B2 / 8;  // 16-byte pieces of the x tile
  static constexpr int kXRegs = (kXPieces + 63) / 64;
  uint4 w[B2 / 32];         // dense: B2/32 chunks; sparse: the first B2/64 hold values
  uint32_t mw[B2 == 256 ? 2 : 1];  // sparse: the lane's metadata words
  uint4 xr[kXRegs > 0 ? kXRegs : 1];  // this lane's share of the x tile (XR = false)
};

// Loads one tile's slab piece (and, without XR, its x columns) into a
// stage.  Every access is a raw buffer load whose resource covers exactly
// the bytes this tile may touch: chunks a sparse tile does not have, the
// metadata of a dense tile, tiles with an out-of-range slot and x rows >= M
// fall outside their resource and read as zero without a memory access.
// The instruction stream is the same for dense and sparse tiles, so loads
// stay in flight across tiles of either kind.
template <int MT, int B2, bool XR>
__device__ __forceinline__ void gemv_load(GemvStage<MT, B2, XR>& st, int32_t ti, int32_t tk,
                                          const uint4* __restrict__ dense,
                                          const uint4* __restrict__ val,
                                          const uint16_t* __restrict__ meta,
                                          const uint16_t* __restrict__ x, const GemvDims& d,
                                          int rs, int lane, int wl) {
  const bool is_dense = ti >= 0;
  const int32_t slot = is_dense ? ti : ~ti;
  const bool ok = is_dense ? (slot < d.n_dense) : (slot < d.n_sparse);
  const int64_t tile = int64_t(d.b1) * B2;  // elements per tile
  const char* wbase = is_dense
      ? reinterpret_cast<const char*>(dense) + (int64_t(slot) * tile + int64_t(rs) * 16 * B2) * 2
      : reinterpret_cast<const char*>(val) + (int64_t(slot) * (tile / 2) + int64_t(rs) * 8 * B2) * 2;
  const int32_t wbytes = ok ? (is_dense ? 32 * B2 : 16 * B2) : 0;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, wbytes);
#pragma unroll
  for (int c = 0; c < B2 / 32; ++c)
    st.w[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, wl * 16 + c * 1024, 0, HYB_W_AUX));
  const char* mbase = reinterpret_cast<const char*>(meta) + (int64_t(slot) * (tile / 16) + int64_t(rs) * B2) * 2;
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(mbase, (ok && !is_dense) ? 2 * B2 : 0);
  if constexpr (B2 == 64) {
    // the aligned dword holding the lane's 16-bit word (a 16-bit load would
    // be zero-extended where it lands, which waits for it there)
    st.mw[0] = __builtin_amdgcn_raw_buffer_load_b32(mr, (wl * 2) & ~3, 0, HYB_M_AUX) >> (16 * (wl & 1));
  } else if constexpr (B2 == 128) {
    st.mw[0] = __builtin_amdgcn_raw_buffer_load_b32(mr, wl * 4, 0, HYB_M_AUX);
  } else {
    const auto mm = __builtin_amdgcn_raw_buffer_load_b64(mr, wl * 8, 0, HYB_M_AUX);
    st.mw[0] = mm[0];
    st.mw[1] = mm[1];
  }
  if constexpr (!XR) {
    // x tile: piece pc = (row m, 8 columns); rows >= M fall outside the resource.
    const __amdgpu_buffer_rsrc_t xrr = make_rsrc(x + int64_t(tk) * B2, ok ? int32_t(d.m * d.ldx * 2) : 0);
#pragma unroll
    for (int i = 0; i < GemvStage<MT, B2, XR>::kXRegs; ++i) {
      const int pc = lane + 64 * i;
      const int m = pc / (B2 / 8);
      const int c8 = pc - m * (B2 / 8);
      const bool valid = pc < GemvStage<MT, B2, XR>::kXPieces && m < d.m;
      const int off = valid ? int(m * d.ldx * 2) + c8 * 16 : 0x7FFFFFF0;
      st.xr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrr, off, 0, 0));
    }
  }
}

// Multiplies one loaded tile into acc.  xs is the tile's x columns in LDS:
// token row m at xs + m * XS (XS = b2 per tile, or kXrTiles * b2 for a staged
// range); without XR this call first stores the stage's x registers there.
template <int MT, int B2, int DT, int META, bool XR>
__device__ __forceinline__ void gemv_compute(const GemvStage<MT, B2, XR>& st, int32_t ti, uint16_t* xs,
                                             const uint4* lut8, const GemvDims& d, int lane,
                                             float (&acc)[MT]) {
  constexpr int XS = XR ? kXrTiles<B2> * B2 : B2;
  const int q = lane >> 4;  // column group of the lane inside a chunk
  if constexpr (!XR) {
    // Stage this tile's x columns in the wavefront's LDS region.  LDS
    // accesses of one wavefront complete in order, so no barrier is needed;
    // the wave barriers keep the compiler from moving LDS accesses across.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < GemvStage<MT, B2, XR>::kXRegs; ++i) {
      const int pc = lane + 64 * i;
      if (pc < GemvStage<MT, B2, XR>::kXPieces) *reinterpret_cast<uint4*>(xs + pc * 8) = st.xr[i];
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (ti >= 0) {
    if (ti >= d.n_dense) return;
#pragma unroll
    for (int c = 0; c < B2 / 32; ++c) {
      const uint4 w = st.w[c];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + m * XS + c * 32 + q * 8);
        float a = acc[m];
        a = dot2<DT>(w.x, xv.x, a);
        a = dot2<DT>(w.y, xv.y, a);
        a = dot2<DT>(w.z, xv.z, a);
        a = dot2<DT>(w.w, xv.w, a);
        acc[m] = a;
      }
    }
  } else {
    if (~ti >= d.n_sparse) return;
    if constexpr (META == HYB_META_MASK8) {
      // 4:8: expand the lane's two groups to their sixteen columns with the
      // selector table, then the dense dot products
#pragma unroll
      for (int c = 0; c < B2 / 64; ++c) {
        const uint4 w = st.w[c];
        const uint32_t word = (st.mw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
        uint32_t e[8];
        expand8_lane(lut8, w.x, w.y, w.z, w.w, word, e);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint16_t* xrow = xs + m * XS + c * 64 + q * 16;
          const uint4 xa = *reinterpret_cast<const uint4*>(xrow);
          const uint4 xb = *reinterpret_cast<const uint4*>(xrow + 8);
          float a = acc[m];
          a = dot2<DT>(e[0], xa.x, a);
          a = dot2<DT>(e[1], xa.y, a);
          a = dot2<DT>(e[2], xa.z, a);
          a = dot2<DT>(e[3], xa.w, a);
          a = dot2<DT>(e[4], xb.x, a);
          a = dot2<DT>(e[5], xb.y, a);
          a = dot2<DT>(e[6], xb.z, a);
          a = dot2<DT>(e[7], xb.w, a);
          acc[m] = a;
        }
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < B2 / 64; ++c) {
      const uint4 w = st.w[c];
      const uint32_t word = (st.mw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
      uint32_t sel[4];
      word_selectors<META>(word, sel);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint16_t* xrow = xs + m * XS + c * 64 + q * 16;
        const uint4 xa = *reinterpret_cast<const uint4*>(xrow);
        const uint4 xb = *reinterpret_cast<const uint4*>(xrow + 8);
        float a = acc[m];
        a = dot2<DT>(w.x, __builtin_amdgcn_perm(xa.y, xa.x, sel[0]), a);
        a = dot2<DT>(w.y, __builtin_amdgcn_perm(xa.w, xa.z, sel[1]), a);
        a = dot2<DT>(w.z, __builtin_amdgcn_perm(xb.y, xb.x, sel[2]), a);
        a = dot2<DT>(w.w, __builtin_amdgcn_perm(xb.w, xb.z, sel[3]), a);
        acc[m] = a;
      }
    }
  }
}

// Decode kernels that have a mixed launch: one token, four wavefronts per
// slab.  (At two and four tokens the mixed launch measured no faster.)
__host__ __device__ constexpr bool gemv_has_halves(int mt, int waves) { return waves == kGemvWaves && mt == 1; }

// The LDS of one decode workgroup.  The kernel declares it and hands it to
// gemv_slab, so that two instantiations of gemv_slab in one kernel (the two
// ring depths of the mixed launch) share one allocation.
template <int MT, int B2, int META, int WAVES, bool XR>
struct GemvSmem {
  static constexpr int XS = XR ? kXrTiles<B2> * B2 : B2;  // x row stride
  uint4 lut8[META == HYB_META_MASK8 ? 256 : 1];
  __attribute__((aligned(16))) uint16_t xs[WAVES][MT * XS];
  float red[WAVES][MT][16];
};

// The product of one 16-row slab (the whole work of one workgroup).  With
// LR the slab also adds the low-rank term sum_j T[m][j] U[row][j] (3BASiL,
// gist.science, section 1: W ~ S + L with L of rank r, here L = U V^T and
// T = X V given): wavefront 0's lanes take row L%16 and every fourth
// 8-column chunk of the rank, and add their partial dot products into the
// row sums before the lane and wavefront reduction, so the order of the
// additions stays fixed.
// With XR the wavefront's whole tile range (at most kXrTiles tiles) has its
// x columns staged once, before the first weight loads.
// With half >= 0 the call takes only rows 8 half .. 8 half + 7 of the
// slab: the other rows' lanes (the four lanes of a row are all in or all
// out) get weight offsets past the end of every resource, so they load
// nothing, and their rows are not stored.  The rows taken see the same
// loads in the same order as with half < 0, so their results are bitwise
// equal.  x comes through the real lane in either case.
template <int MT, int B2, int DT, int META, int WAVES, int STAGES, bool LR = false, bool XR = false>
__device__ __forceinline__ void gemv_slab(const uint4* __restrict__ dense, const uint4* __restrict__ val,
                                          const uint16_t* __restrict__ meta, const int32_t* __restrict__ tidx,
                                          const uint16_t* __restrict__ x, void* __restrict__ y,
                                          const GemvDims& d, int64_t slab,
                                          GemvSmem<MT, B2, META, WAVES, XR>& sm, int half = -1) {
  constexpr int XS = GemvSmem<MT, B2, META, WAVES, XR>::XS;
  uint4* lut8 = sm.lut8;
  if constexpr (META == HYB_META_MASK8) {
    fill_expand8_lut(lut8);
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slabs_per_tile = d.b1 / 16;
  const int64_t tn = slab / slabs_per_tile;
  const int rs = int(slab - tn * slabs_per_tile);
  const int32_t tk0 = (wave * d.tiles_k) / WAVES;
  const int32_t cnt = ((wave + 1) * d.tiles_k) / WAVES - tk0;
  const int32_t* __restrict__ trow = tidx + tn * d.tiles_k + tk0;
  uint16_t* xs = sm.xs[wave];
  const int ln = (half < 0 || ((lane & 15) >> 3) == half) ? lane : (1 << 22);

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;

  // Tiles past the end of the range get the index kNone: its slot is out
  // of range, so the loads for it cover zero bytes and the loop body issues
  // the same loads on every trip.
  constexpr int32_t kNone = INT32_MIN;
  auto tile_index = [&](int32_t j) -> int32_t { return j < cnt ? trow[j] : kNone; };
  // STAGES-deep register ring: while a tile is multiplied, the loads of
  // the next STAGES-1 tiles are in flight.  The inner loop is fully
  // unrolled so every stage index is a compile-time constant.
  GemvStage<MT, B2, XR> st[STAGES];
  int32_t ti[STAGES];
  // XR: the range's x columns, row m at x + m ldx + tk0 b2 (cnt b2 values),
  // as 1 KiB loads issued before anything else; rows >= M read as zero.
  constexpr int kXrLoads = XR ? kXrTiles<B2> * B2 * 2 / 1024 : 1;
  uint4 xv[XR ? MT : 1][kXrLoads];
  if constexpr (XR) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const __amdgpu_buffer_rsrc_t xr =
          make_rsrc(x + int64_t(m) * d.ldx + int64_t(tk0) * B2, m < d.m ? cnt * B2 * 2 : 0);
#pragma unroll
      for (int i = 0; i < kXrLoads; ++i)
        xv[m][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, i * 1024 + lane * 16, 0, HYB_M_AUX));
    }
  }
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    ti[s] = tile_index(s);
    gemv_load<MT, B2, XR>(st[s], ti[s], tk0 + s, dense, val, meta, x, d, rs, lane, ln);
  }
  if constexpr (XR) {
    // the x loads were issued first, so waiting for them does not wait for
    // the weights in flight behind them
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < kXrLoads; ++i) *reinterpret_cast<uint4*>(xs + m * XS + i * 512 + lane * 8) = xv[m][i];
    __builtin_amdgcn_wave_barrier();
  }
  int32_t tiN = tile_index(STAGES - 1);
  for (int32_t i = 0; i < cnt; i += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      constexpr int kLast = STAGES - 1;
      const int ld = (s + kLast) % STAGES;
      ti[ld] = tiN;
      gemv_load<MT, B2, XR>(st[ld], tiN, tk0 + i + s + kLast, dense, val, meta, x, d, rs, lane, ln);
      tiN = tile_index(i + s + STAGES);
      if (i + s < cnt)
        gemv_compute<MT, B2, DT, META, XR>(st[s], ti[s], XR ? xs + (i + s) * B2 : xs, lut8, d, lane, acc);
    }
  }

  if constexpr (LR) {
    if (wave == 0) {
      const int64_t row = slab * 16 + (lane & 15);
      for (int32_t j0 = (lane >> 4) * 8; j0 < d.rank; j0 += 32) {
        const uint4 uv = *reinterpret_cast<const uint4*>(d.u + row * d.ldu + j0);
        const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
        float uf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uf[2 * i] = widen16<DT>(uw[i] & 0xFFFFu);
          uf[2 * i + 1] = widen16<DT>(uw[i] >> 16);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < d.m) {
            const float4 t0 = *reinterpret_cast<const float4*>(d.t + int64_t(m) * d.ldt + j0);
            const float4 t1 = *reinterpret_cast<const float4*>(d.t + int64_t(m) * d.ldt + j0 + 4);
            float a = acc[m];
            a = fmaf(uf[0], t0.x, a);
            a = fmaf(uf[1], t0.y, a);
            a = fmaf(uf[2], t0.z, a);
            a = fmaf(uf[3], t0.w, a);
            a = fmaf(uf[4], t1.x, a);
            a = fmaf(uf[5], t1.y, a);
            a = fmaf(uf[6], t1.z, a);
            a = fmaf(uf[7], t1.w, a);
            acc[m] = a;
          }
        }
      }
    }
  }

  // Lanes L, L^16, L^32, L^48 share row L%16: swizzle-add across the two
  // 16-lane halves of each 32-lane group, then across the 32-lane halves.
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float v = acc[m];
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    v += __shfl_xor(v, 32);
    acc[m] = v;
  }
  if (lane < 16) {
#pragma unroll
    for (int m = 0; m < MT; ++m) sm.red[wave][m][lane] = acc[m];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < MT * 16; i += blockDim.x) {
    const int m = i >> 4, r = i & 15;
    if (m < d.m && (half < 0 || (r >> 3) == half)) {
      float v = sm.red[0][m][r];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) v += sm.red[w][m][r];
      store_out(y, d.ydt, int64_t(m) * d.ldy + slab * 16 + r, v);
    }
  }
}

template <int MT, int B2, int DT, int META, int WAVES, int STAGES, bool LR, bool XR>
__global__ __launch_bounds__(64 * WAVES) void k_gemv(const uint4* __restrict__ dense,
                                                     const uint4* __restrict__ val,
                                                     const uint16_t* __restrict__ meta,
                                                     const int32_t* __restrict__ tidx,
                                                     const uint16_t* __restrict__ x,
                                                     void* __restrict__ y, GemvDims d) {
  __shared__ GemvSmem<MT, B2, META, WAVES, XR> sm;
  gemv_slab<MT, B2, DT, META, WAVES, STAGES, LR, XR>(dense, val, meta, tidx, x, y, d, blockIdx.x, sm);
}

// The mixed launch: workgroups below full take whole slabs as k_gemv does;
// the others are half slabs, slab full + (b - full) / 2, half (b - full) % 2,
// with a ring one stage deeper, which keeps as many weight bytes in flight
// per workgroup as a whole slab with the shallower ring.  A kernel of its
// own, because the deeper ring's registers would lower k_gemv's occupancy
// where no slab is split.
template <int MT, int B2, int DT, int META, int WAVES, int STAGES, bool LR, bool XR>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_mixed(const uint4* __restrict__ dense,
                                                           const uint4* __restrict__ val,
                                                           const uint16_t* __restrict__ meta,
                                                           const int32_t* __restrict__ tidx,
                                                           const uint16_t* __restrict__ x,
                                                           void* __restrict__ y, GemvDims d, int32_t full) {
  __shared__ GemvSmem<MT, B2, META, WAVES, XR> sm;
  const int32_t b = blockIdx.x;
  if (b < full) {
    gemv_slab<MT, B2, DT, META, WAVES, STAGES, LR, XR>(dense, val, meta, tidx, x, y, d, b, sm);
  } else {
    gemv_slab<MT, B2, DT, META, WAVES, STAGES + 1, LR, XR>(dense, val, meta, tidx, x, y, d,
                                                           full + ((b - full) >> 1), sm, (b - full) & 1);
  }
}

// Grouped decode product: one launch multiplies the same x by up to
// kMaxGroup matrices (for instance the q, k and v projections of a layer,
// each with its own tile map and sparsity).  Matrix g owns workgroups
// slab_start[g] .. slab_start[g+1]-1, one per 16-row slab as above, so every
// slab runs exactly the single-matrix code and the results are bitwise those
// of separate launches.
struct GemvGroup {
  const uint4* dense[kMaxGroup];
  const uint4* val[kMaxGroup];
  const uint16_t* meta[kMaxGroup];
  const int32_t* tidx[kMaxGroup];
  void* y[kMaxGroup];
  int64_t ldy[kMaxGroup];
  int32_t n_dense[kMaxGroup], n_sparse[kMaxGroup], b1[kMaxGroup];
  int32_t slab_start[kMaxGroup + 1];
  int32_t count;
};

template <int MT, int B2, int DT, int META, int WAVES, int STAGES, bool XR>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_grouped(const uint16_t* __restrict__ x, GemvDims d,
                                                             GemvGroup g) {
  const int32_t b = blockIdx.x;
  int gi = 0;
  for (int i = 1; i < g.count; ++i) gi = b >= g.slab_start[i] ? i : gi;
  d.ldy = g.ldy[gi];
  d.n_dense = g.n_dense[gi];
  d.n_sparse = g.n_sparse[gi];
  d.b1 = g.b1[gi];
  __shared__ GemvSmem<MT, B2, META, WAVES, XR> sm;
  gemv_slab<MT, B2, DT, META, WAVES, STAGES, false, XR>(g.dense[gi], g.val[gi], g.meta[gi], g.tidx[gi], x, g.y[gi], d,
                                                        b - g.slab_start[gi], sm);
}

}  // namespace


namespace {

// Up to this many tokens the decode kernel can stage x per wavefront range.
constexpr int kXrMaxM = 2;

// Whether the decode kernel stages x once per wavefront range: few tokens,
// four wavefronts per slab, and every range within kXrTiles tiles (so
// k <= 4 * 2048 columns at any b2).
bool gemv_xr(int64_t tiles_k, int b2, int waves, int m) {
  const int64_t max_tiles = b2 == 64 ? kXrTiles<64> : b2 == 128 ? kXrTiles<128> : kXrTiles<256>;
  return m <= kXrMaxM && waves == kGemvWaves && (tiles_k + waves - 1) / waves <= max_tiles;
}

// Workgroups of k_gemv_mixed one CU holds at once (0 if the query fails),
// taken once per instantiation: every device this library runs on is gfx950.
template <int MT, int B2, int DT, int META, int W, bool LR, bool XR>
int gemv_mixed_per_cu() {
  static const int n = [] {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &v, reinterpret_cast<const void*>(k_gemv_mixed<MT, B2, DT, META, W, kGemvStages, LR, XR>), 64 * W, 0) !=
        hipSuccess) {
      (void)hipGetLastError();
      v = 0;
    }
    return v;
  }();
  return n;
}

// One decode launch over `slabs` slabs.  Where full < slabs and the kernel
// has the half body, the mixed launch (full whole slabs, 2 (slabs - full)
// halves) runs if all its workgroups are resident at once; otherwise k_gemv
// over whole slabs.
template <int MT, int B2, int DT, int META, bool LR, int W, bool XR>
void gemv_launch(int64_t slabs, int64_t full, hipStream_t s, const GemvPtrs& q, const GemvDims& d) {
  const dim3 block(64 * W);
  if constexpr (gemv_has_halves(MT, W)) {
    const int64_t wgs = full + 2 * (slabs - full);
    if (full < slabs && wgs <= int64_t(gemv_mixed_per_cu<MT, B2, DT, META, W, LR, XR>()) * device_cus()) {
      hipLaunchKernelGGL((k_gemv_mixed<MT, B2, DT, META, W, kGemvStages, LR, XR>), dim3(unsigned(wgs)), block, 0, s,
                         q.dense, q.val, q.meta, q.tidx, q.x, q.y, d, int32_t(full));
      return;
    }
  }
  hipLaunchKernelGGL((k_gemv<MT, B2, DT, META, W, kGemvStages, LR, XR>), dim3(unsigned(slabs)), block, 0, s, q.dense,
                     q.val, q.meta, q.tidx, q.x, q.y, d);
}

template <int MT, int DT, int META, bool LR, int W, bool XR = false>
void gemv_b2(int b2, int64_t slabs, int64_t full, hipStream_t s, const GemvPtrs& q, const GemvDims& d) {
  switch (b2) {
    case 64:
      return gemv_launch<MT, 64, DT, META, LR, W, XR>(slabs, full, s, q, d);
    case 128:
      return gemv_launch<MT, 128, DT, META, LR, W, XR>(slabs, full, s, q, d);
    default:
      return gemv_launch<MT, 256, DT, META, LR, W, XR>(slabs, full, s, q, d);
  }
}

// MT-token variant with the wavefront count of gemv_waves; x staged per
// wavefront range (XR) where gemv_xr allows it.
template <int MT, int DT, int META, bool LR>
void gemv_w(int waves, bool xr, int b2, int64_t slabs, int64_t full, hipStream_t s, const GemvPtrs& q,
            const GemvDims& d) {
  if constexpr (MT <= 4) {
    if (waves == 8) return gemv_b2<MT, DT, META, LR, 8>(b2, slabs, slabs, s, q, d);
  } else {
    if (waves == 16) return gemv_b2<MT, DT, META, LR, 16>(b2, slabs, slabs, s, q, d);
  }
  if constexpr (MT <= kXrMaxM) {
    if (xr) return gemv_b2<MT, DT, META, LR, kGemvWaves, true>(b2, slabs, full, s, q, d);
  }
  gemv_b2<MT, DT, META, LR, kGemvWaves>(b2, slabs, full, s, q, d);
}

template <int DT, int META, bool LR>
void gemv_mt(int m, int waves, bool xr, int b2, int64_t slabs, int64_t full, hipStream_t s, const GemvPtrs& q,
             const GemvDims& d) {
  if (m <= 1) gemv_w<1, DT, META, LR>(waves, xr, b2, slabs, full, s, q, d);
  else if (m <= 2) gemv_w<2, DT, META, LR>(waves, xr, b2, slabs, full, s, q, d);
  else if (m <= 4) gemv_w<4, DT, META, LR>(waves, xr, b2, slabs, full, s, q, d);
  else if (m <= 8) gemv_w<8, DT, META, LR>(waves, xr, b2, slabs, full, s, q, d);
  else gemv_w<16, DT, META, LR>(waves, xr, b2, slabs, full, s, q, d);
}

}  // namespace

namespace {

template <bool LR>
hipError_t launch_gemv_impl(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                            void* y, int y_dtype, int64_t ldy, const float* t, int64_t ldt, const void* u,
                            int64_t ldu, int rank, hipStream_t s) {
  GemvPtrs q{static_cast<const uint4*>(P.dense), static_cast<const uint4*>(P.val),
             static_cast<const uint16_t*>(P.meta), P.tidx, static_cast<const uint16_t*>(x), y};
  GemvDims d{};
  d.ldx = ldx;
  d.ldy = ldy;
  d.tiles_k = int32_t(L.tiles_k);
  d.n_dense = int32_t(L.n_dense);
  d.n_sparse = int32_t(L.n_sparse);
  d.b1 = L.b1;
  d.m = m;
  d.ydt = y_dtype;
  d.t = t;
  d.ldt = ldt;
  d.u = static_cast<const uint16_t*>(u);
  d.ldu = ldu;
  d.rank = rank;
  const int64_t slabs = L.n / 16;
  const int w = gemv_waves(slabs, m);
  const bool xr = gemv_xr(L.tiles_k, L.b2, w, m);
  // slabs the last round may run as halves (only kernels with the half
  // body, and only where the mixed launch fits, take them)
  const int64_t full = gemv_full_slabs(slabs, device_cus());
  if (L.dtype == HYB_BF16) {
    if (L.meta == HYB_META_IDX2) gemv_mt<HYB_BF16, HYB_META_IDX2, LR>(m, w, xr, L.b2, slabs, full, s, q, d);
    else if (L.meta == HYB_META_MASK4) gemv_mt<HYB_BF16, HYB_META_MASK4, LR>(m, w, xr, L.b2, slabs, full, s, q, d);
    else gemv_mt<HYB_BF16, HYB_META_MASK8, LR>(m, w, xr, L.b2, slabs, full, s, q, d);
  } else {
    if (L.meta == HYB_META_IDX2) gemv_mt<HYB_F16, HYB_META_IDX2, LR>(m, w, xr, L.b2, slabs, full, s, q, d);
    else if (L.meta == HYB_META_MASK4) gemv_mt<HYB_F16, HYB_META_MASK4, LR>(m, w, xr, L.b2, slabs, full, s, q, d);
    else gemv_mt<HYB_F16, HYB_META_MASK8, LR>(m, w, xr, L.b2, slabs, full, s, q, d);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                       void* y, int y_dtype, int64_t ldy, hipStream_t s) {
  return launch_gemv_impl<false>(L, P, x, m, ldx, y, y_dtype, ldy, nullptr, 0, nullptr, 0, 0, s);
}


hipError_t launch_gemv_lowrank(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                               const float* t, int64_t ldt, const void* u, int64_t ldu, int rank, void* y,
                               int y_dtype, int64_t ldy, hipStream_t s) {
  return launch_gemv_impl<true>(L, P, x, m, ldx, y, y_dtype, ldy, t, ldt, u, ldu, rank, s);
}

namespace {

template <int MT, int DT, int META, int W, bool XR = false>
void gemv_grouped_b2(int b2, dim3 grid, hipStream_t s, const uint16_t* x, const GemvDims& d, const GemvGroup& g) {
  const dim3 block(64 * W);
  switch (b2) {
    case 64:
      hipLaunchKernelGGL((k_gemv_grouped<MT, 64, DT, META, W, kGemvStages, XR>), grid, block, 0, s, x, d, g);
      break;
    case 128:
      hipLaunchKernelGGL((k_gemv_grouped<MT, 128, DT, META, W, kGemvStages, XR>), grid, block, 0, s, x, d, g);
      break;
    default:
      hipLaunchKernelGGL((k_gemv_grouped<MT, 256, DT, META, W, kGemvStages, XR>), grid, block, 0, s, x, d, g);
      break;
  }
}

template <int MT, int DT, int META>
void gemv_grouped_w(int waves, bool xr, int b2, dim3 grid, hipStream_t s, const uint16_t* x, const GemvDims& d,
                    const GemvGroup& g) {
  if constexpr (MT <= 4) {
    if (waves == 8) return gemv_grouped_b2<MT, DT, META, 8>(b2, grid, s, x, d, g);
  } else {
    if (waves == 16) return gemv_grouped_b2<MT, DT, META, 16>(b2, grid, s, x, d, g);
  }
  if constexpr (MT <= kXrMaxM) {
    if (xr) return gemv_grouped_b2<MT, DT, META, kGemvWaves, true>(b2, grid, s, x, d, g);
  }
  gemv_grouped_b2<MT, DT, META, kGemvWaves>(b2, grid, s, x, d, g);
}

template <int DT, int META>
void gemv_grouped_mt(int m, int waves, bool xr, int b2, dim3 grid, hipStream_t s, const uint16_t* x,
                     const GemvDims& d, const GemvGroup& g) {
  if (m <= 1) gemv_grouped_w<1, DT, META>(waves, xr, b2, grid, s, x, d, g);
  else if (m <= 2) gemv_grouped_w<2, DT, META>(waves, xr, b2, grid, s, x, d, g);
  else if (m <= 4) gemv_grouped_w<4, DT, META>(waves, xr, b2, grid, s, x, d, g);
  else if (m <= 8) gemv_grouped_w<8, DT, META>(waves, xr, b2, grid, s, x, d, g);
  else gemv_grouped_w<16, DT, META>(waves, xr, b2, grid, s, x, d, g);
}

}  // namespace

hipError_t launch_gemv_grouped(int count, const hyb_layout* L, const hyb_packed* P, const void* x, int m,
                               int64_t ldx, void* const* y, int y_dtype, const int64_t* ldy, hipStream_t s) {
  // Each matrix runs with the wavefront count hyb_gemv would give it on its
  // own (so its result is bitwise that of a separate launch): one launch
  // per distinct count, at most two.
  int waves[kMaxGroup];
  for (int i = 0; i < count; ++i) waves[i] = gemv_waves(L[i].n / 16, m);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  bool done[kMaxGroup] = {};
  for (int first = 0; first < count; ++first) {
    if (done[first]) continue;
    const int w = waves[first];
    GemvGroup g{};
    int64_t slabs = 0;
    for (int i = first; i < count; ++i) {
      if (done[i] || waves[i] != w) continue;
      done[i] = true;
      const int c = g.count++;
      g.dense[c] = static_cast<const uint4*>(P[i].dense);
      g.val[c] = static_cast<const uint4*>(P[i].val);
      g.meta[c] = static_cast<const uint16_t*>(P[i].meta);
      g.tidx[c] = P[i].tidx;
      g.y[c] = y[i];
      g.ldy[c] = ldy[i];
      g.n_dense[c] = int32_t(L[i].n_dense);
      g.n_sparse[c] = int32_t(L[i].n_sparse);
      g.b1[c] = L[i].b1;
      g.slab_start[c] = int32_t(slabs);
      slabs += L[i].n / 16;
    }
    g.slab_start[g.count] = int32_t(slabs);
    if (slabs == 0) continue;
    GemvDims d{};
    d.ldx = ldx;
    d.tiles_k = int32_t(L[0].tiles_k);
    d.m = m;
    d.ydt = y_dtype;
    const dim3 grid(static_cast<unsigned>(slabs));
    const bool xr = gemv_xr(L[0].tiles_k, L[0].b2, w, m);
    if (L[0].dtype == HYB_BF16) {
      if (L[0].meta == HYB_META_IDX2) gemv_grouped_mt<HYB_BF16, HYB_META_IDX2>(m, w, xr, L[0].b2, grid, s, xp, d, g);
      else if (L[0].meta == HYB_META_MASK4) gemv_grouped_mt<HYB_BF16, HYB_META_MASK4>(m, w, xr, L[0].b2, grid, s, xp, d, g);
      else gemv_grouped_mt<HYB_BF16, HYB_META_MASK8>(m, w, xr, L[0].b2, grid, s, xp, d, g);
    } else {
      if (L[0].meta == HYB_META_IDX2) gemv_grouped_mt<HYB_F16, HYB_META_IDX2>(m, w, xr, L[0].b2, grid, s, xp, d, g);
      else if (L[0].meta == HYB_META_MASK4) gemv_grouped_mt<HYB_F16, HYB_META_MASK4>(m, w, xr, L[0].b2, grid, s, xp, d, g);
      else gemv_grouped_mt<HYB_F16, HYB_META_MASK8>(m, w, xr, L[0].b2, grid, s, xp, d, g);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace hyb
