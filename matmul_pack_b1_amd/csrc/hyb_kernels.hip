// HIP kernels for gfx950 (MI355X): pack, unpack, decode GEMV and the
// matrix-core GEMM over the HYB1 tile-hybrid dense / 2:4 stream format.
//
// Format (see include/hyb.h): every 1 KiB of the dense or value stream is a
// piece of one 16-row slab of one tile, and lane L (0..63) of a wavefront
// owns 16 bytes of it:
//   dense chunk  = 16 rows x 32 columns; lane L: row L%16, columns 8*(L/16)..+7
//   value chunk  = 16 rows x 64 columns (32 stored values per row); lane L:
//                  row L%16, the four groups 4*(L/16)..+3, two values each
//   metadata     = one 16-bit word per (value chunk, lane), a lane's words
//                  for the b2/64 chunks of a slab back to back.
// A wavefront therefore streams each slab with fully coalesced 16-byte loads,
// and the dense chunk is also the A-operand layout of the 16x16x32 MFMA.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hyb_internal.h"

// Tuning knobs of the decode kernel (defaults chosen by measurement):
// wavefronts per workgroup splitting a slab's tile columns, tiles kept in
// flight per wavefront, and the cache-policy bits of the weight loads.
#ifndef HYB_GEMV_WAVES
#define HYB_GEMV_WAVES 4
#endif
#ifndef HYB_GEMV_STAGES
#define HYB_GEMV_STAGES 2
#endif
#ifndef HYB_W_AUX
#define HYB_W_AUX 2  // non-temporal: the weights are read once per product
#endif

namespace hyb {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 half8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// ------------------------------------------------------------- helpers ----

template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  // Two exact products summed into c in fp32 (v_dot2c_f32_{bf16,f16}).
  if constexpr (DT == HYB_BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  c, false);
  }
}

template <int DT>
__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
  if constexpr (DT == HYB_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
}

// fp32 -> 16-bit with round-to-nearest-even (NaN stays NaN).
template <int DT>
__device__ __forceinline__ uint16_t round16(float v) {
  if constexpr (DT == HYB_BF16) {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
    return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  }
}

__device__ __forceinline__ void store_out(void* y, int ydt, int64_t idx, float v) {
  if (ydt == HYB_F32) {
    static_cast<float*>(y)[idx] = v;
  } else if (ydt == HYB_BF16) {
    static_cast<uint16_t*>(y)[idx] = round16<HYB_BF16>(v);
  } else {
    static_cast<uint16_t*>(y)[idx] = round16<HYB_F16>(v);
  }
}

// Kept pair of one group of four 16-bit values: rank by magnitude key
// (bits & 0x7FFF), larger first, ties to the lower position; keep the first
// two.  Returns the 4-bit mask of kept positions.
__device__ __forceinline__ uint32_t kept_mask(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3) {
  const uint32_t k0 = ((v0 & 0x7FFFu) << 2) | 3u;
  const uint32_t k1 = ((v1 & 0x7FFFu) << 2) | 2u;
  const uint32_t k2 = ((v2 & 0x7FFFu) << 2) | 1u;
  const uint32_t k3 = ((v3 & 0x7FFFu) << 2) | 0u;
  // rank = number of strictly larger scores (scores are distinct)
  const uint32_t r0 = (k1 > k0) + (k2 > k0) + (k3 > k0);
  const uint32_t r1 = (k0 > k1) + (k2 > k1) + (k3 > k1);
  const uint32_t r2 = (k0 > k2) + (k1 > k2) + (k3 > k2);
  const uint32_t r3 = (k0 > k3) + (k1 > k3) + (k2 > k3);
  return (r0 < 2 ? 1u : 0u) | (r1 < 2 ? 2u : 0u) | (r2 < 2 ? 4u : 0u) | (r3 < 2 ? 8u : 0u);
}

// Kept positions (i0, i1) of one nibble.  Always in [0, 4]; an invalid
// nibble gives unspecified positions but never an out-of-range index.
__device__ __forceinline__ void nibble_positions(uint32_t nib, int meta, uint32_t& i0, uint32_t& i1) {
  if (meta == HYB_META_IDX2) {
    i0 = nib & 3u;
    i1 = (nib >> 2) & 3u;
  } else {
    i0 = __builtin_ctz(nib | 0x10u);
    i1 = 31u - __builtin_clz(nib | 1u);
  }
}

template <int META>
__device__ __forceinline__ void nibble_positions_t(uint32_t nib, uint32_t& i0, uint32_t& i1) {
  if constexpr (META == HYB_META_IDX2) {
    i0 = nib & 3u;
    i1 = (nib >> 2) & 3u;
  } else {
    i0 = __builtin_ctz(nib | 0x10u);
    i1 = 31u - __builtin_clz(nib | 1u);
  }
}

// v_perm selector that gathers the 16-bit elements i0 and i1 of the 64-bit
// pair {hi:lo} into one dword (i0 in the low half).
__device__ __forceinline__ uint32_t gather_selector(uint32_t i0, uint32_t i1) {
  return 0x01000100u + i0 * 0x0202u + (i1 * 0x0202u << 16);
}

// v_perm selector placing the stored pair (lo = value at i0, hi = value at
// i1) into elements e, e+1 of a dense group; other elements are zero.
__device__ __forceinline__ uint32_t scatter_selector(uint32_t e, uint32_t i0, uint32_t i1) {
  const uint32_t s0 = (e == i1) ? 0x0302u : (e == i0) ? 0x0100u : 0x0C0Cu;
  const uint32_t s1 = (e + 1 == i1) ? 0x0302u : (e + 1 == i0) ? 0x0100u : 0x0C0Cu;
  return s0 | (s1 << 16);
}

// ---------------------------------------------------------------- pack ----

struct PackParams {
  const uint16_t* w;
  int64_t ldw;
  uint16_t* dense;
  uint16_t* val;
  uint16_t* meta;  // 16-bit words
  const int32_t* tidx;
  int64_t tiles_k, n_dense, n_sparse;
  int b1, meta_kind;
};

// One workgroup = one tile x four 16-row slabs; wavefront w packs slab
// (blockIdx.y * 4 + w).
template <int B2>
__global__ __launch_bounds__(256) void k_pack(PackParams p) {
  const int lane = threadIdx.x & 63;
  const int rs = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int64_t t = blockIdx.x;
  const int64_t tn = t / p.tiles_k, tk = t - tn * p.tiles_k;
  const int32_t ti = p.tidx[t];
  const int64_t row = tn * p.b1 + rs * 16 + (lane & 15);
  const uint16_t* wrow = p.w + row * p.ldw + tk * B2;
  const int64_t tile = int64_t(p.b1) * B2;
  if (ti >= 0) {
    if (ti >= p.n_dense) return;
    uint16_t* dst = p.dense + ti * tile + int64_t(rs) * 16 * B2 + lane * 8;
#pragma unroll
    for (int c = 0; c < B2 / 32; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(wrow + c * 32 + (lane >> 4) * 8);
      *reinterpret_cast<uint4*>(dst + c * 512) = v;
    }
    return;
  }
  const int64_t s = ~int64_t(ti);
  if (s >= p.n_sparse) return;
  uint16_t* vdst = p.val + s * (tile / 2) + int64_t(rs) * 8 * B2 + lane * 8;
  uint32_t words[B2 / 64];
#pragma unroll
  for (int c = 0; c < B2 / 64; ++c) {
    const uint16_t* src = wrow + c * 64 + (lane >> 4) * 16;
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
    const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t outv[4];
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = d[2 * q], hi = d[2 * q + 1];
      const uint32_t e[4] = {lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu, hi >> 16};
      const uint32_t mask = kept_mask(e[0], e[1], e[2], e[3]);
      const uint32_t i0 = __builtin_ctz(mask);
      const uint32_t i1 = 31u - __builtin_clz(mask);
      // select elements i0, i1 (both in 0..3)
      const uint32_t v0 = i0 == 0 ? e[0] : i0 == 1 ? e[1] : i0 == 2 ? e[2] : e[3];
      const uint32_t v1 = i1 == 0 ? e[0] : i1 == 1 ? e[1] : i1 == 2 ? e[2] : e[3];
      outv[q] = v0 | (v1 << 16);
      const uint32_t nib = (p.meta_kind == HYB_META_IDX2) ? (i0 | (i1 << 2)) : mask;
      word |= nib << (4 * q);
    }
    *reinterpret_cast<uint4*>(vdst + c * 512) = make_uint4(outv[0], outv[1], outv[2], outv[3]);
    words[c] = word;
  }
  uint16_t* mdst = p.meta + s * (tile / 16) + int64_t(rs) * B2 + lane * (B2 / 64);
  if constexpr (B2 == 64) {
    mdst[0] = uint16_t(words[0]);
  } else if constexpr (B2 == 128) {
    *reinterpret_cast<uint32_t*>(mdst) = words[0] | (words[1] << 16);
  } else {
    *reinterpret_cast<uint2*>(mdst) = make_uint2(words[0] | (words[1] << 16), words[2] | (words[3] << 16));
  }
}

// -------------------------------------------------------------- unpack ----

template <int B2>
__global__ __launch_bounds__(256) void k_unpack(PackParams p) {
  const int lane = threadIdx.x & 63;
  const int rs = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int64_t t = blockIdx.x;
  const int64_t tn = t / p.tiles_k, tk = t - tn * p.tiles_k;
  const int32_t ti = p.tidx[t];
  const int64_t row = tn * p.b1 + rs * 16 + (lane & 15);
  uint16_t* wrow = const_cast<uint16_t*>(p.w) + row * p.ldw + tk * B2;
  const int64_t tile = int64_t(p.b1) * B2;
  if (ti >= 0) {
    if (ti >= p.n_dense) return;
    const uint16_t* src = p.dense + ti * tile + int64_t(rs) * 16 * B2 + lane * 8;
#pragma unroll
    for (int c = 0; c < B2 / 32; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c * 512);
      *reinterpret_cast<uint4*>(wrow + c * 32 + (lane >> 4) * 8) = v;
    }
    return;
  }
  const int64_t s = ~int64_t(ti);
  if (s >= p.n_sparse) return;
  const uint16_t* vsrc = p.val + s * (tile / 2) + int64_t(rs) * 8 * B2 + lane * 8;
  const uint16_t* msrc = p.meta + s * (tile / 16) + int64_t(rs) * B2 + lane * (B2 / 64);
#pragma unroll
  for (int c = 0; c < B2 / 64; ++c) {
    const uint4 v = *reinterpret_cast<const uint4*>(vsrc + c * 512);
    const uint32_t word = msrc[c];
    const uint32_t pv[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t i0, i1;
      nibble_positions((word >> (4 * q)) & 0xFu, p.meta_kind, i0, i1);
      o[2 * q] = __builtin_amdgcn_perm(0u, pv[q], scatter_selector(0, i0, i1));
      o[2 * q + 1] = __builtin_amdgcn_perm(0u, pv[q], scatter_selector(2, i0, i1));
    }
    uint16_t* dst = wrow + c * 64 + (lane >> 4) * 16;
    *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// ---------------------------------------------------------------- GEMV ----
//
// y[m, n] = sum_k W'[n, k] x[m, k] for m < M <= 16.
// One workgroup = one 16-row slab; its WAVES wavefronts split the tile
// columns of the slab's tile row into contiguous ranges.  Per tile a
// wavefront loads the slab piece (dense: b2/32 x 16 B per lane; sparse: b2/64
// x 16 B of values plus b2/64 16-bit metadata words per lane) and this tile's
// x columns (MT x b2), stages x in its own LDS region, and accumulates in
// fp32 with v_dot2.  Sparse groups gather their two x values with one v_perm
// each.  Loads run one tile ahead through a two-stage register ring (the
// loop is unrolled by two so no in-flight register is ever copied).  Lanes
// L, L^16, L^32, L^48 hold the same row and are combined with cross-lane
// swizzles; the wavefronts are then summed in a fixed order through LDS, so
// results are reproducible run to run.

struct GemvDims {
  int64_t ldx, ldy;
  int32_t tiles_k, n_dense, n_sparse;
  int b1, m, ydt;
};

constexpr int kBufDword3 = 0x00020000;  // raw buffer resource word 3 on gfx9-family parts

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufDword3);
}

template <int MT, int B2>
struct GemvStage {
  static constexpr int kXPieces = MT * B2 / 8;  // 16-byte pieces of the x tile
  static constexpr int kXRegs = (kXPieces + 63) / 64;
  uint4 w[B2 / 32];         // dense: B2/32 chunks; sparse: the first B2/64 hold values
  uint32_t mw[B2 == 256 ? 2 : 1];  // sparse: the lane's metadata words
  uint4 xr[kXRegs];         // this lane's share of the x tile
};

// Loads one tile's slab piece and x columns into a stage.  Every access is
// a raw buffer load whose resource covers exactly the bytes this tile may
// touch: chunks a sparse tile does not have, the metadata of a dense tile,
// tiles with an out-of-range slot and x rows >= M fall outside their
// resource and read as zero without a memory access.  The instruction
// stream is the same for dense and sparse tiles, so loads stay in flight
// across tiles of either kind.
template <int MT, int B2>
__device__ __forceinline__ void gemv_load(GemvStage<MT, B2>& st, int32_t ti, int32_t tk,
                                          const uint4* __restrict__ dense,
                                          const uint4* __restrict__ val,
                                          const uint16_t* __restrict__ meta,
                                          const uint16_t* __restrict__ x, const GemvDims& d,
                                          int rs, int lane) {
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
    st.w[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, lane * 16 + c * 1024, 0, HYB_W_AUX));
  const char* mbase = reinterpret_cast<const char*>(meta) + (int64_t(slot) * (tile / 16) + int64_t(rs) * B2) * 2;
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(mbase, (ok && !is_dense) ? 2 * B2 : 0);
  if constexpr (B2 == 64) {
    st.mw[0] = __builtin_amdgcn_raw_buffer_load_b16(mr, lane * 2, 0, 0);
  } else if constexpr (B2 == 128) {
    st.mw[0] = __builtin_amdgcn_raw_buffer_load_b32(mr, lane * 4, 0, 0);
  } else {
    const auto mm = __builtin_amdgcn_raw_buffer_load_b64(mr, lane * 8, 0, 0);
    st.mw[0] = mm[0];
    st.mw[1] = mm[1];
  }
  // x tile: piece pc = (row m, 8 columns); rows >= M fall outside the resource.
  const __amdgpu_buffer_rsrc_t xrr = make_rsrc(x + int64_t(tk) * B2, ok ? int32_t(d.m * d.ldx * 2) : 0);
#pragma unroll
  for (int i = 0; i < GemvStage<MT, B2>::kXRegs; ++i) {
    const int pc = lane + 64 * i;
    const int m = pc / (B2 / 8);
    const int c8 = pc - m * (B2 / 8);
    const bool valid = pc < GemvStage<MT, B2>::kXPieces && m < d.m;
    const int off = valid ? int(m * d.ldx * 2) + c8 * 16 : 0x7FFFFFF0;
    st.xr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrr, off, 0, 0));
  }
}

template <int MT, int B2, int DT, int META>
__device__ __forceinline__ void gemv_compute(const GemvStage<MT, B2>& st, int32_t ti, uint16_t* xs,
                                             const GemvDims& d, int lane, float (&acc)[MT]) {
  const int q = lane >> 4;  // column group of the lane inside a chunk
  // Stage this tile's x columns in the wavefront's LDS region.  LDS
  // accesses of one wavefront complete in order, so no barrier is needed;
  // the wave barriers keep the compiler from moving LDS accesses across.
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < GemvStage<MT, B2>::kXRegs; ++i) {
    const int pc = lane + 64 * i;
    if (pc < GemvStage<MT, B2>::kXPieces) *reinterpret_cast<uint4*>(xs + pc * 8) = st.xr[i];
  }
  __builtin_amdgcn_wave_barrier();
  if (ti >= 0) {
    if (ti >= d.n_dense) return;
#pragma unroll
    for (int c = 0; c < B2 / 32; ++c) {
      const uint4 w = st.w[c];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + m * B2 + c * 32 + q * 8);
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
#pragma unroll
    for (int c = 0; c < B2 / 64; ++c) {
      const uint4 w = st.w[c];
      const uint32_t word = (st.mw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
      uint32_t sel[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t i0, i1;
        nibble_positions_t<META>((word >> (4 * g)) & 0xFu, i0, i1);
        sel[g] = gather_selector(i0, i1);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint16_t* xrow = xs + m * B2 + c * 64 + q * 16;
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

template <int MT, int B2, int DT, int META, int WAVES, int STAGES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv(const uint4* __restrict__ dense,
                                                     const uint4* __restrict__ val,
                                                     const uint16_t* __restrict__ meta,
                                                     const int32_t* __restrict__ tidx,
                                                     const uint16_t* __restrict__ x,
                                                     void* __restrict__ y, GemvDims d) {
  __shared__ __attribute__((aligned(16))) uint16_t xs_all[WAVES][MT * B2];
  __shared__ float red[WAVES][MT][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t slab = blockIdx.x;
  const int slabs_per_tile = d.b1 / 16;
  const int64_t tn = slab / slabs_per_tile;
  const int rs = int(slab - tn * slabs_per_tile);
  const int32_t tk0 = (wave * d.tiles_k) / WAVES;
  const int32_t cnt = ((wave + 1) * d.tiles_k) / WAVES - tk0;
  const int32_t* __restrict__ trow = tidx + tn * d.tiles_k + tk0;
  uint16_t* xs = xs_all[wave];

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
  GemvStage<MT, B2> st[STAGES];
  int32_t ti[STAGES];
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    ti[s] = tile_index(s);
    gemv_load<MT, B2>(st[s], ti[s], tk0 + s, dense, val, meta, x, d, rs, lane);
  }
  int32_t tiN = tile_index(STAGES - 1);
  for (int32_t i = 0; i < cnt; i += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      constexpr int kLast = STAGES - 1;
      const int ld = (s + kLast) % STAGES;
      ti[ld] = tiN;
      gemv_load<MT, B2>(st[ld], tiN, tk0 + i + s + kLast, dense, val, meta, x, d, rs, lane);
      tiN = tile_index(i + s + STAGES);
      if (i + s < cnt) gemv_compute<MT, B2, DT, META>(st[s], ti[s], xs, d, lane, acc);
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
    for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < MT * 16; i += blockDim.x) {
    const int m = i >> 4, r = i & 15;
    if (m < d.m) {
      float v = red[0][m][r];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) v += red[w][m][r];
      store_out(y, d.ydt, int64_t(m) * d.ldy + slab * 16 + r, v);
    }
  }
}

// ---------------------------------------------------------------- GEMM ----
//
// Y[m, n] = sum_k X[m, k] W'[n, k] for any M, on 16x16x32 MFMA.
// Workgroup tile 128 (n) x 128 (m), 4 wavefronts in a 2 x 2 grid, each
// 64 (n) x 64 (m) = 4 x 4 MFMA blocks.  The k loop walks 64-column blocks.
// A operands (W') come straight from the streams into registers -- a dense
// chunk already is the A layout; a sparse chunk is expanded in registers
// with v_perm to the 16 columns its lane owns, and the B operand (X, staged
// in LDS, double buffered) is read with the matching column permutation, so
// the products are those of W' in any case.

struct GemmParams {
  const uint4* dense;
  const uint4* val;
  const uint16_t* meta;
  const int32_t* tidx;
  const uint16_t* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  int64_t n, tiles_k, n_dense, n_sparse;
  int b1, m, ydt, meta_kind;
};

constexpr int kGemmBN = 128, kGemmBM = 128, kGemmBK = 64;
constexpr int kXsStride = kGemmBK + 8;  // padded LDS row (elements)

template <int B2, int DT>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kGemmBM * kXsStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int q = lane >> 4;
  const int64_t n0 = int64_t(blockIdx.x) * kGemmBN + wn * 64;  // first row of this wave
  const int64_t m0 = int64_t(blockIdx.y) * kGemmBM;
  const bool rows_ok = n0 < p.n;
  const int64_t tn = n0 / p.b1;
  const int rs0 = int((n0 - tn * p.b1) / 16);
  const int32_t* trow = p.tidx + tn * p.tiles_k;
  constexpr int kb_per_tile = B2 / kGemmBK;
  const int64_t steps = p.tiles_k * kb_per_tile;
  const int64_t dense_tile = int64_t(p.b1) * B2 / 8;
  const int64_t val_tile = int64_t(p.b1) * B2 / 16;
  const int64_t meta_tile = int64_t(p.b1) * B2 / 16;

  // raw A data for one k step: 4 slabs x (2 dense chunks | 1 value chunk + word)
  struct ARaw {
    uint4 a[4][2];
    uint32_t word[4];
    int kind;  // 0 dense, 1 sparse, 2 skip
  };

  auto load_a = [&](int64_t step, ARaw& r) {
    const int64_t tk = step / kb_per_tile;
    const int kb = int(step - tk * kb_per_tile);
    const int32_t ti = rows_ok ? __builtin_amdgcn_readfirstlane(trow[tk]) : 0;
    r.kind = 2;
    if (!rows_ok) return;
    if (ti >= 0) {
      if (ti >= p.n_dense) return;
      r.kind = 0;
      const uint4* src = p.dense + ti * dense_tile + lane;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
        for (int h = 0; h < 2; ++h) r.a[sl][h] = src[(int64_t(rs0 + sl) * 2 * B2) + (2 * kb + h) * 64];
      }
    } else {
      const int64_t s = ~int64_t(ti);
      if (s >= p.n_sparse) return;
      r.kind = 1;
      const uint4* src = p.val + s * val_tile + lane;
      const uint16_t* msrc = p.meta + s * meta_tile + lane * (B2 / 64) + kb;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        r.a[sl][0] = src[int64_t(rs0 + sl) * B2 + kb * 64];
        r.word[sl] = msrc[int64_t(rs0 + sl) * B2];
      }
    }
  };

  // X tile for one k step: 128 rows x 64 columns = 1024 pieces of 16 B.
  auto load_x = [&](int64_t step, uint4 (&xr)[4]) {
    const int64_t k0 = step * kGemmBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + 256 * i;
      const int r = pc >> 3, c8 = pc & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + r < p.m) v = *reinterpret_cast<const uint4*>(p.x + (m0 + r) * p.ldx + k0 + c8 * 8);
      xr[i] = v;
    }
  };
  auto store_x = [&](int buf, const uint4 (&xr)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + 256 * i;
      const int r = pc >> 3, c8 = pc & 7;
      *reinterpret_cast<uint4*>(&xs[buf][r * kXsStride + c8 * 8]) = xr[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  ARaw anext;
  uint4 xr[4];
  if (steps > 0) {
    load_a(0, anext);
    load_x(0, xr);
    store_x(0, xr);
  }
  __syncthreads();

  for (int64_t step = 0; step < steps; ++step) {
    const int buf = int(step & 1);
    ARaw acur = anext;
    if (step + 1 < steps) {
      load_a(step + 1, anext);
      load_x(step + 1, xr);
    }
    if (acur.kind != 2) {
      uint4 a[4][2];
      if (acur.kind == 0) {
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          a[sl][0] = acur.a[sl][0];
          a[sl][1] = acur.a[sl][1];
        }
      } else {
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const uint4 v = acur.a[sl][0];
          const uint32_t pv[4] = {v.x, v.y, v.z, v.w};
          uint32_t o[8];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint32_t i0, i1;
            nibble_positions((acur.word[sl] >> (4 * g)) & 0xFu, p.meta_kind, i0, i1);
            o[2 * g] = __builtin_amdgcn_perm(0u, pv[g], scatter_selector(0, i0, i1));
            o[2 * g + 1] = __builtin_amdgcn_perm(0u, pv[g], scatter_selector(2, i0, i1));
          }
          a[sl][0] = make_uint4(o[0], o[1], o[2], o[3]);
          a[sl][1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
      }
      // B operand column offset of this lane for MFMA half h:
      // dense chunk h covers columns 32h + 8q..+7; expanded sparse half h
      // covers columns 16q + 8h..+7.
      const int kofs0 = acur.kind == 0 ? q * 8 : q * 16;
      const int kstep = acur.kind == 0 ? 32 : 8;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const uint16_t* xrow = &xs[buf][(wm * 64 + mb * 16 + (lane & 15)) * kXsStride];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint4 b = *reinterpret_cast<const uint4*>(xrow + kofs0 + h * kstep);
#pragma unroll
          for (int sl = 0; sl < 4; ++sl) acc[sl][mb] = mfma16x16x32<DT>(a[sl][h], b, acc[sl][mb]);
        }
      }
    }
    if (step + 1 < steps) store_x(buf ^ 1, xr);
    __syncthreads();
  }

  if (!rows_ok) return;
  // acc[sl][mb] lane L holds rows n0 + 16 sl + 4 (L/16) + 0..3 of token
  // m0 + 64 wm + 16 mb + L%16.
  const bool vec_ok = (p.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.y) & 15) == 0);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int64_t m = m0 + wm * 64 + mb * 16 + (lane & 15);
    if (m >= p.m) continue;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int64_t n = n0 + sl * 16 + q * 4;
      const f32x4_t v = acc[sl][mb];
      const int64_t base = m * p.ldy + n;
      if (p.ydt == HYB_F32) {
        float* dst = static_cast<float*>(p.y) + base;
        if (vec_ok) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = v[e];
        }
      } else {
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = p.ydt == HYB_BF16 ? round16<HYB_BF16>(v[e]) : round16<HYB_F16>(v[e]);
        uint16_t* dst = static_cast<uint16_t*>(p.y) + base;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = o[e];
      }
    }
  }
}

}  // namespace

// -------------------------------------------------------------- launchers -

hipError_t launch_pack(const hyb_layout& L, const void* w, int64_t ldw, const hyb_packed& P,
                       hipStream_t s) {
  PackParams p{};
  p.w = static_cast<const uint16_t*>(w);
  p.ldw = ldw;
  p.dense = static_cast<uint16_t*>(P.dense);
  p.val = static_cast<uint16_t*>(P.val);
  p.meta = static_cast<uint16_t*>(P.meta);
  p.tidx = P.tidx;
  p.tiles_k = L.tiles_k;
  p.n_dense = L.n_dense;
  p.n_sparse = L.n_sparse;
  p.b1 = L.b1;
  p.meta_kind = L.meta;
  const dim3 grid(unsigned(L.tiles_n * L.tiles_k), unsigned(L.b1 / 64));
  switch (L.b2) {
    case 64: hipLaunchKernelGGL(k_pack<64>, grid, dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL(k_pack<128>, grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL(k_pack<256>, grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_unpack(const hyb_layout& L, const hyb_packed& P, void* w, int64_t ldw,
                         hipStream_t s) {
  PackParams p{};
  p.w = static_cast<const uint16_t*>(w);
  p.ldw = ldw;
  p.dense = static_cast<uint16_t*>(P.dense);
  p.val = static_cast<uint16_t*>(P.val);
  p.meta = static_cast<uint16_t*>(P.meta);
  p.tidx = P.tidx;
  p.tiles_k = L.tiles_k;
  p.n_dense = L.n_dense;
  p.n_sparse = L.n_sparse;
  p.b1 = L.b1;
  p.meta_kind = L.meta;
  const dim3 grid(unsigned(L.tiles_n * L.tiles_k), unsigned(L.b1 / 64));
  switch (L.b2) {
    case 64: hipLaunchKernelGGL(k_unpack<64>, grid, dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL(k_unpack<128>, grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL(k_unpack<256>, grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

namespace {

constexpr int kGemvWaves = HYB_GEMV_WAVES;
constexpr int kGemvStages = HYB_GEMV_STAGES;

struct GemvPtrs {
  const uint4* dense;
  const uint4* val;
  const uint16_t* meta;
  const int32_t* tidx;
  const uint16_t* x;
  void* y;
};

template <int MT, int DT, int META>
void gemv_b2(int b2, dim3 grid, hipStream_t s, const GemvPtrs& q, const GemvDims& d) {
  const dim3 block(64 * kGemvWaves);
  switch (b2) {
    case 64:
      hipLaunchKernelGGL((k_gemv<MT, 64, DT, META, kGemvWaves, kGemvStages>), grid, block, 0, s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d);
      break;
    case 128:
      hipLaunchKernelGGL((k_gemv<MT, 128, DT, META, kGemvWaves, kGemvStages>), grid, block, 0, s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d);
      break;
    default:
      hipLaunchKernelGGL((k_gemv<MT, 256, DT, META, kGemvWaves, kGemvStages>), grid, block, 0, s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d);
      break;
  }
}

template <int DT, int META>
void gemv_mt(int m, int b2, dim3 grid, hipStream_t s, const GemvPtrs& q, const GemvDims& d) {
  if (m <= 1) gemv_b2<1, DT, META>(b2, grid, s, q, d);
  else if (m <= 2) gemv_b2<2, DT, META>(b2, grid, s, q, d);
  else if (m <= 4) gemv_b2<4, DT, META>(b2, grid, s, q, d);
  else if (m <= 8) gemv_b2<8, DT, META>(b2, grid, s, q, d);
  else gemv_b2<16, DT, META>(b2, grid, s, q, d);
}

}  // namespace

hipError_t launch_gemv(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                       void* y, int y_dtype, int64_t ldy, hipStream_t s) {
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
  const dim3 grid(unsigned(L.n / 16));
  if (L.dtype == HYB_BF16) {
    if (L.meta == HYB_META_IDX2) gemv_mt<HYB_BF16, HYB_META_IDX2>(m, L.b2, grid, s, q, d);
    else gemv_mt<HYB_BF16, HYB_META_MASK4>(m, L.b2, grid, s, q, d);
  } else {
    if (L.meta == HYB_META_IDX2) gemv_mt<HYB_F16, HYB_META_IDX2>(m, L.b2, grid, s, q, d);
    else gemv_mt<HYB_F16, HYB_META_MASK4>(m, L.b2, grid, s, q, d);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                       void* y, int y_dtype, int64_t ldy, hipStream_t s) {
  GemmParams p{};
  p.dense = static_cast<const uint4*>(P.dense);
  p.val = static_cast<const uint4*>(P.val);
  p.meta = static_cast<const uint16_t*>(P.meta);
  p.tidx = P.tidx;
  p.x = static_cast<const uint16_t*>(x);
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  p.n = L.n;
  p.tiles_k = L.tiles_k;
  p.n_dense = L.n_dense;
  p.n_sparse = L.n_sparse;
  p.b1 = L.b1;
  p.m = m;
  p.ydt = y_dtype;
  p.meta_kind = L.meta;
  const int64_t gm = (int64_t(m) + kGemmBM - 1) / kGemmBM;
  if (gm > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid(unsigned((L.n + kGemmBN - 1) / kGemmBN), unsigned(gm));
  if (L.dtype == HYB_BF16) {
    switch (L.b2) {
      case 64: hipLaunchKernelGGL((k_gemm<64, HYB_BF16>), grid, dim3(256), 0, s, p); break;
      case 128: hipLaunchKernelGGL((k_gemm<128, HYB_BF16>), grid, dim3(256), 0, s, p); break;
      default: hipLaunchKernelGGL((k_gemm<256, HYB_BF16>), grid, dim3(256), 0, s, p); break;
    }
  } else {
    switch (L.b2) {
      case 64: hipLaunchKernelGGL((k_gemm<64, HYB_F16>), grid, dim3(256), 0, s, p); break;
      case 128: hipLaunchKernelGGL((k_gemm<128, HYB_F16>), grid, dim3(256), 0, s, p); break;
      default: hipLaunchKernelGGL((k_gemm<256, HYB_F16>), grid, dim3(256), 0, s, p); break;
    }
  }
  return hipGetLastError();
}

}  // namespace hyb
