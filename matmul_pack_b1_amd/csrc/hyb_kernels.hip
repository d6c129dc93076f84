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

#include <atomic>
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
// The GEMM re-reads each weight slab once per token block, so its weight
// loads keep the default cache policy (the decode kernel's are
// non-temporal: it reads each weight once).
#ifndef HYB_GEMM_W_NT
#define HYB_GEMM_W_NT 0
#endif
#ifndef HYB_GEMM_GROUP_N
#define HYB_GEMM_GROUP_N 4
#endif
#ifndef HYB_GEMM_C192
#define HYB_GEMM_C192 0.8
#endif
#ifndef HYB_GEMM_C_RX
#define HYB_GEMM_C_RX 0.29
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
typedef __attribute__((ext_vector_type(16))) __bf16 bf16x16_t;
typedef __attribute__((ext_vector_type(16))) _Float16 half16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;  // an LDS-resident vector

// ------------------------------------------------------------- helpers ----

// fp32 value of a bf16 / fp16 bit pattern (low 16 bits of `bits`).
template <int DT>
__device__ __forceinline__ float widen16(uint32_t bits) {
  if constexpr (DT == HYB_BF16) {
    return __builtin_bit_cast(float, bits << 16);
  } else {
    return float(__builtin_bit_cast(_Float16, uint16_t(bits)));
  }
}

// Bits of a where m is set, of b elsewhere.
__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

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

// 4:8 groups (metadata kind HYB_META_MASK8): eight aligned columns keep
// four values, stored in ascending position as the 64-bit pair
// {v3 v2 : v1 v0}, with a mask byte (bit p = position p kept).
// Kept mask of eight 16-bit values: the same ranking as kept_mask (key
// bits & 0x7FFF, larger first, ties to the lower position), first four kept.
__device__ __forceinline__ uint32_t kept_mask8(const uint32_t (&e)[8]) {
  uint32_t sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sc[i] = ((e[i] & 0x7FFFu) << 3) | uint32_t(7 - i);
  uint32_t mask = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t r = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) r += (j != i && sc[j] > sc[i]) ? 1u : 0u;
    mask |= (r < 4 ? 1u : 0u) << i;
  }
  return mask;
}

// v_perm selector that writes positions 2j and 2j+1 of a 4:8 group from its
// stored pair: the value of rank r (number of kept positions below) for a
// kept position, zero otherwise.  A mask without exactly four bits gives
// unspecified values, never an out-of-range access.
__device__ __forceinline__ uint32_t expand8_selector(uint32_t mask, int j) {
  uint32_t out = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = 2 * j + h;
    const uint32_t r = __builtin_popcount(mask & ((1u << p) - 1u));
    const uint32_t sel = ((mask >> p) & 1u) ? (0x0100u + 0x0202u * r) : 0x0C0Cu;
    out |= sel << (16 * h);
  }
  return out;
}

// Selector table of every mask byte, one 16-byte entry (j = 0..3) per mask,
// filled once per workgroup into LDS by its threads.
__device__ __forceinline__ void fill_expand8_lut(uint4* lut) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x)
    lut[i] = make_uint4(expand8_selector(i, 0), expand8_selector(i, 1), expand8_selector(i, 2),
                        expand8_selector(i, 3));
}

// The sixteen columns of one lane's two 4:8 groups as eight dwords
// (positions 2j, 2j+1 in dword j; group 1 in dwords 4..7), from the lane's
// 16-byte value piece and its 16-bit metadata word.
__device__ __forceinline__ void expand8_lane(const uint4* lut, uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                             uint32_t word, uint32_t (&e)[8]) {
  const uint4 s0 = lut[word & 0xFFu];
  const uint4 s1 = lut[(word >> 8) & 0xFFu];
  e[0] = __builtin_amdgcn_perm(v1, v0, s0.x);
  e[1] = __builtin_amdgcn_perm(v1, v0, s0.y);
  e[2] = __builtin_amdgcn_perm(v1, v0, s0.z);
  e[3] = __builtin_amdgcn_perm(v1, v0, s0.w);
  e[4] = __builtin_amdgcn_perm(v3, v2, s1.x);
  e[5] = __builtin_amdgcn_perm(v3, v2, s1.y);
  e[6] = __builtin_amdgcn_perm(v3, v2, s1.z);
  e[7] = __builtin_amdgcn_perm(v3, v2, s1.w);
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
    if (p.meta_kind == HYB_META_MASK8) {
      // two groups of eight: four kept values each, in ascending position
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t e[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[2 * i] = d[4 * h + i] & 0xFFFFu;
          e[2 * i + 1] = d[4 * h + i] >> 16;
        }
        const uint32_t mask = kept_mask8(e);
        uint32_t kv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t r = __builtin_popcount(mask & ((1u << i) - 1u));
#pragma unroll
          for (int t = 0; t < 4; ++t) kv[t] = (((mask >> i) & 1u) && r == uint32_t(t)) ? e[i] : kv[t];
        }
        outv[2 * h] = kv[0] | (kv[1] << 16);
        outv[2 * h + 1] = kv[2] | (kv[3] << 16);
        word |= mask << (8 * h);
      }
      *reinterpret_cast<uint4*>(vdst + c * 512) = make_uint4(outv[0], outv[1], outv[2], outv[3]);
      words[c] = word;
      continue;
    }
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

// The slab's 16 rows are assembled row-major in a wavefront-private LDS
// buffer (LDS accesses of one wavefront complete in order, so no barrier is
// needed; the wave barrier keeps the compiler from moving them), then
// stored as whole row segments: each store instruction writes 1 KiB of
// contiguous row bytes instead of 64-byte halves of 16 rows.
template <int B2>
__global__ __launch_bounds__(256) void k_unpack(PackParams p) {
  constexpr int kRow = B2 + 8;  // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) uint16_t stage[4][16 * kRow];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int rs = blockIdx.y * 4 + wv;
  const int64_t t = blockIdx.x;
  const int64_t tn = t / p.tiles_k, tk = t - tn * p.tiles_k;
  const int32_t ti = p.tidx[t];
  const int r = lane & 15, q = lane >> 4;
  uint16_t* buf = stage[wv];
  const int64_t tile = int64_t(p.b1) * B2;
  if (ti >= 0) {
    if (ti >= p.n_dense) return;
    const uint16_t* src = p.dense + ti * tile + int64_t(rs) * 16 * B2 + lane * 8;
#pragma unroll
    for (int c = 0; c < B2 / 32; ++c)
      *reinterpret_cast<uint4*>(buf + r * kRow + c * 32 + q * 8) = *reinterpret_cast<const uint4*>(src + c * 512);
  } else {
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
      if (p.meta_kind == HYB_META_MASK8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[j] = __builtin_amdgcn_perm(v.y, v.x, expand8_selector(word & 0xFFu, j));
          o[4 + j] = __builtin_amdgcn_perm(v.w, v.z, expand8_selector(word >> 8, j));
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t i0, i1;
          nibble_positions((word >> (4 * g)) & 0xFu, p.meta_kind, i0, i1);
          o[2 * g] = __builtin_amdgcn_perm(0u, pv[g], scatter_selector(0, i0, i1));
          o[2 * g + 1] = __builtin_amdgcn_perm(0u, pv[g], scatter_selector(2, i0, i1));
        }
      }
      uint16_t* dst = buf + r * kRow + c * 64 + q * 16;
      *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
  __builtin_amdgcn_wave_barrier();
  constexpr int kLanesPerRow = B2 / 8;             // 16-byte pieces per row
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
  const int rr = lane / kLanesPerRow, cc = (lane % kLanesPerRow) * 8;
  uint16_t* wbase = const_cast<uint16_t*>(p.w) + (tn * p.b1 + rs * 16) * p.ldw + tk * B2 + cc;
#pragma unroll
  for (int i = 0; i < 16 / kRowsPerStore; ++i) {
    const int row = i * kRowsPerStore + rr;
    *reinterpret_cast<uint4*>(wbase + int64_t(row) * p.ldw) = *reinterpret_cast<const uint4*>(buf + row * kRow + cc);
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
// fp32 with v_dot2.  Sparse 2:4 groups gather their two x values with one
// v_perm each; 4:8 groups are expanded to their eight columns with v_perm
// selectors from a per-workgroup LDS table of all 256 mask bytes.  Loads run one tile ahead through a two-stage register ring (the
// loop is unrolled by two so no in-flight register is ever copied).  Lanes
// L, L^16, L^32, L^48 hold the same row and are combined with cross-lane
// swizzles; the wavefronts are then summed in a fixed order through LDS, so
// results are reproducible run to run.

struct GemvDims {
  int64_t ldx, ldy;
  int32_t tiles_k, n_dense, n_sparse;
  int b1, m, ydt;
  // low-rank term T U^T (hyb_gemv_lowrank only): T m x rank fp32, U n x rank
  const float* t;
  const uint16_t* u;
  int64_t ldt, ldu;
  int32_t rank;
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
                                             const uint4* lut8, const GemvDims& d, int lane,
                                             float (&acc)[MT]) {
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
          const uint16_t* xrow = xs + m * B2 + c * 64 + q * 16;
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

// The product of one 16-row slab (the whole work of one workgroup).  With
// LR the slab also adds the low-rank term sum_j T[m][j] U[row][j] (3BASiL,
// gist.science, section 1: W ~ S + L with L of rank r, here L = U V^T and
// T = X V given): wavefront 0's lanes take row L%16 and every fourth
// 8-column chunk of the rank, and add their partial dot products into the
// row sums before the lane and wavefront reduction, so the order of the
// additions stays fixed.
template <int MT, int B2, int DT, int META, int WAVES, int STAGES, bool LR = false>
__device__ __forceinline__ void gemv_slab(const uint4* __restrict__ dense, const uint4* __restrict__ val,
                                          const uint16_t* __restrict__ meta, const int32_t* __restrict__ tidx,
                                          const uint16_t* __restrict__ x, void* __restrict__ y,
                                          const GemvDims& d, int64_t slab) {
  __shared__ __attribute__((aligned(16))) uint16_t xs_all[WAVES][MT * B2];
  __shared__ float red[WAVES][MT][16];
  __shared__ uint4 lut8[META == HYB_META_MASK8 ? 256 : 1];
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
      if (i + s < cnt) gemv_compute<MT, B2, DT, META>(st[s], ti[s], xs, lut8, d, lane, acc);
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

template <int MT, int B2, int DT, int META, int WAVES, int STAGES, bool LR>
__global__ __launch_bounds__(64 * WAVES) void k_gemv(const uint4* __restrict__ dense,
                                                     const uint4* __restrict__ val,
                                                     const uint16_t* __restrict__ meta,
                                                     const int32_t* __restrict__ tidx,
                                                     const uint16_t* __restrict__ x,
                                                     void* __restrict__ y, GemvDims d) {
  gemv_slab<MT, B2, DT, META, WAVES, STAGES, LR>(dense, val, meta, tidx, x, y, d, blockIdx.x);
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

template <int MT, int B2, int DT, int META, int WAVES, int STAGES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_grouped(const uint16_t* __restrict__ x, GemvDims d,
                                                             GemvGroup g) {
  const int32_t b = blockIdx.x;
  int gi = 0;
  for (int i = 1; i < g.count; ++i) gi = b >= g.slab_start[i] ? i : gi;
  d.ldy = g.ldy[gi];
  d.n_dense = g.n_dense[gi];
  d.n_sparse = g.n_sparse[gi];
  d.b1 = g.b1[gi];
  gemv_slab<MT, B2, DT, META, WAVES, STAGES>(g.dense[gi], g.val[gi], g.meta[gi], g.tidx[gi], x, g.y[gi], d,
                                              b - g.slab_start[gi]);
}

// ---------------------------------------------------------------- GEMM ----
//
// Y[m, n] = sum_k X[m, k] W'[n, k] for any M on the matrix cores
// (k_gemm_rx up to 128 tokens, k_gemm_lds above).  A K step is 64 columns
// and a wavefront's unit is 64 weight rows (four 16-row slabs).  A sparse
// slab piece is one v_smfmac_*_16x16x64 A operand (32 kept values per row)
// with its 2-bit indices: the stored value chunk and its idx2 word are
// exactly that instruction's operand layout, so sparse tiles run on the
// sparse matrix cores with no expansion.  Both kinds take the same B
// operands (X[m][8q..8q+7] and X[m][32+8q..32+8q+7] for lane group q).
// Partial sums are always added in a fixed order, so results are
// reproducible.

struct GemmDims {
  int64_t ldx, ldy;
  int32_t n, m, tiles_k, n_dense, n_sparse;
  int b1, ydt;
  // low-rank term T U^T (hyb_gemm_lowrank; rank 0 otherwise): T m x rank
  // fp32, U n x rank of the weight dtype
  const float* t;
  const uint16_t* u;
  int64_t ldt, ldu;
  int32_t rank;
};

// Adds the low-rank term sum_j U[row][j] T[tok][j] (3BASiL, gist.science,
// section 1: W ~ S + L with L = U V^T, and T = X V) to a block of 16 x 16
// accumulator tiles: slab s holds rows row0 + 16 s, token block b tokens
// tok0 + 16 b (lane L: rows 4 (L/16) + 0..3 of the slab, token L%16), the
// layout of the products above.  Per 32-wide slice of the rank each slab's
// U piece and each token block's T piece is loaded once.  With bf16
// weights T is split into bf16 hi + lo (|T - hi - lo| <= 2^-16 |T|) and
// each tile takes two exact 16x16x32 products; with fp16 weights (where a
// 16-bit T could overflow) the fp32 16x16x4 instruction takes the products,
// lane group q supplying j = j0 + 8q + e to step e of both operands.  Rows
// are whole (n is a multiple of 64); tokens >= m and j >= rank read as zero.
template <int DT, int NS, int NT>
__device__ __forceinline__ void lr_block(f32x4_t (&c)[NS][NT], const GemmDims& d, int64_t row0, int64_t tok0,
                                         int lane) {
  const int q = lane >> 4, r = lane & 15;
  for (int32_t j0 = 0; j0 < d.rank; j0 += 32) {
    const int32_t j = j0 + 8 * q;
    const bool j_ok = j < d.rank;
    uint4 uw[NS];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
      uw[sl] = j_ok ? *reinterpret_cast<const uint4*>(d.u + (row0 + 16 * sl + r) * d.ldu + j)
                    : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int64_t tok = tok0 + 16 * b + r;
      float4 t0 = make_float4(0.f, 0.f, 0.f, 0.f), t1 = t0;
      if (j_ok && tok < d.m) {
        t0 = *reinterpret_cast<const float4*>(d.t + tok * d.ldt + j);
        t1 = *reinterpret_cast<const float4*>(d.t + tok * d.ldt + j + 4);
      }
      const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
      if constexpr (DT == HYB_BF16) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t h0 = round16<HYB_BF16>(tv[2 * e]), h1 = round16<HYB_BF16>(tv[2 * e + 1]);
          const uint32_t l0 = round16<HYB_BF16>(tv[2 * e] - widen16<HYB_BF16>(h0));
          const uint32_t l1 = round16<HYB_BF16>(tv[2 * e + 1] - widen16<HYB_BF16>(h1));
          hi[e] = h0 | (h1 << 16);
          lo[e] = l0 | (l1 << 16);
        }
        const uint4 bh = make_uint4(hi[0], hi[1], hi[2], hi[3]), bl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          c[sl][b] = mfma16x16x32<HYB_BF16>(uw[sl], bh, c[sl][b]);
          c[sl][b] = mfma16x16x32<HYB_BF16>(uw[sl], bl, c[sl][b]);
        }
      } else {
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          const uint32_t w4[4] = {uw[sl].x, uw[sl].y, uw[sl].z, uw[sl].w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            c[sl][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(widen16<DT>(e & 1 ? w4[e >> 1] >> 16 : w4[e >> 1] & 0xFFFFu),
                                                            tv[e], c[sl][b], 0, 0, 0);
        }
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ f32x4_t smfmac16x16x64(uint4 a, uint4 b0, uint4 b1, uint32_t idx, f32x4_t c) {
  const uint32_t bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  if constexpr (DT == HYB_BF16) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                     __builtin_bit_cast(bf16x16_t, bb), c, idx, 0, 0);
  } else {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(half8_t, a),
                                                    __builtin_bit_cast(half16_t, bb), c, idx, 0, 0);
  }
}

// 2-bit index word (i0 | i1 << 2 per group) from a metadata word.
template <int META>
__device__ __forceinline__ uint32_t idx2_word(uint32_t word) {
  if constexpr (META == HYB_META_MASK8) {
    return 0u;  // 4:8 groups have no 2-bit index word; their paths never ask
  } else if constexpr (META == HYB_META_IDX2) {
    return word & 0xFFFFu;
  } else {
    uint32_t out = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t i0, i1;
      nibble_positions_t<HYB_META_MASK4>((word >> (4 * g)) & 0xFu, i0, i1);
      out |= ((i0 & 3u) | ((i1 & 3u) << 2)) << (4 * g);
    }
    return out;
  }
}

// --------------------------------------------------- GEMM (register-fed) --
//
// Memory-bound range (17 to a few hundred tokens): the weights must stream
// at the decode kernel's rate while the tokens are multiplied on the matrix
// cores.  A workgroup owns 64 weight rows (four 16-row slabs) and BM = 16*MB
// tokens; its WAVES wavefronts split the K steps into contiguous ranges, as
// the decode kernel's do, and never synchronise inside the K walk.  Each
// lane loads exactly its operands straight into a STAGES-deep register
// ring: its slab pieces and, from L2, its B operands
// X[m][8q..8q+7] and X[m][32+8q..32+8q+7] of every token block.  Past the
// end of a wavefront's range, or past the last token row, the loads fall
// outside the buffer resources and read zero, so every trip issues the same
// loads.  At the end the wavefronts' partial sums are added through LDS in
// a fixed tree order (reproducible results).
// One step's operands for one lane: per slab two 16-byte weight pieces (the
// two halves of a dense piece's 2:4 split, or the sparse chunk and zeros)
// and the aligned dword holding the sparse metadata word (a 16-bit load is
// zero-extended by the compiler where it lands, which waits for it and
// drains the ring); the B operands of every token block; the tile index.
template <int MB, int RG>
struct GemmRxStage {
  u32x4_t v0[RG][4], v1[RG][4];
  uint32_t m[RG][4];
  uint4 b[MB][2];
  int32_t ti[RG];
};

// With four wavefronts and up to 64 tokens the launch bound asks for two
// wavefronts per SIMD (at most 256 registers each), so that two workgroups
// share a CU; 128 tokens, or two row groups per wavefront, need the whole
// register file of a SIMD.  RG is the number of 64-row groups per
// workgroup (each wavefront multiplies all of them over its K range: two
// groups halve the X reads per weight byte).
template <int B2, int DT, int META, int MB, int WAVES, int STAGES, int RG>
__global__ __launch_bounds__(64 * WAVES, (WAVES == 4 && MB <= 4 && RG == 1) ? 2 : 1) void k_gemm_rx(
    const uint4* __restrict__ dense, const uint4* __restrict__ val, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ tidx, const uint16_t* __restrict__ x, void* __restrict__ y, GemmDims d) {
  static_assert(WAVES == 4 || WAVES == 8, "tree reduction over 4 or 8 wavefronts");
  constexpr int BM = 16 * MB;
  constexpr int kStepsPerTile = B2 / 64;
  constexpr int kPart = RG * 4 * MB * 64 * 4;  // floats of one wavefront's partial sums
  __shared__ __attribute__((aligned(16))) float red[WAVES / 2][kPart];
  __shared__ uint4 lut8[META == HYB_META_MASK8 ? 256 : 1];
  if constexpr (META == HYB_META_MASK8) {
    fill_expand8_lut(lut8);
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int r = lane & 15;
  const int32_t n0 = int32_t(blockIdx.x) * 64 * RG;
  const int32_t m0 = int32_t(blockIdx.y) * BM;
  const int32_t steps = d.tiles_k * kStepsPerTile;
  const int32_t s0 = (wave * steps) / WAVES;
  const int32_t cnt = ((wave + 1) * steps) / WAVES - s0;
  const int32_t mrows = d.m - m0 < BM ? d.m - m0 : BM;
  const int64_t tile = int64_t(d.b1) * B2;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + int64_t(m0) * d.ldx, mrows * int32_t(d.ldx) * 2);
  // Lane L's 2:4 operand of a dense slab covers columns 16q..16q+15 of the
  // step: lane groups 2(q%2) and 2(q%2)+1 of dense chunk q/2.
  const int dense_off = (q >> 1) * 1024 + ((2 * (q & 1)) * 16 + r) * 16;

  constexpr int32_t kNone = INT32_MIN;
  auto load = [&](GemmRxStage<MB, RG>& st, int32_t it) {
    const bool live = it < cnt;
    const int kb = (s0 + it) % kStepsPerTile;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int32_t ng = n0 + 64 * g;
      const bool rows = ng < d.n;
      const int32_t tn = rows ? ng / d.b1 : 0;
      const int rs0 = (ng - tn * d.b1) / 16;
      int32_t ti = (live && rows) ? tidx[int64_t(tn) * d.tiles_k + (s0 + it) / kStepsPerTile] : kNone;
      const bool is_dense = ti >= 0;
      const int32_t slot = is_dense ? ti : ~ti;
      if (is_dense ? (slot >= d.n_dense) : (slot >= d.n_sparse)) ti = kNone;
      st.ti[g] = ti;
      const bool ok = ti != kNone;
      const int32_t slab_bytes = is_dense ? 32 * B2 : 16 * B2;
      const char* base = is_dense
          ? reinterpret_cast<const char*>(dense) + (int64_t(slot) * tile + int64_t(rs0) * 16 * B2) * 2
          : reinterpret_cast<const char*>(val) + (int64_t(slot) * (tile / 2) + int64_t(rs0) * 8 * B2) * 2;
      const __amdgpu_buffer_rsrc_t ar = make_rsrc(ok ? base : nullptr, ok ? 4 * slab_bytes : 0);
      const char* mbase = reinterpret_cast<const char*>(meta) + (int64_t(slot) * (tile / 16) + int64_t(rs0) * B2) * 2;
      const __amdgpu_buffer_rsrc_t mr =
          make_rsrc((ok && !is_dense) ? mbase : nullptr, (ok && !is_dense) ? 8 * B2 : 0);
      const int32_t o0 = is_dense ? 2 * kb * 1024 + dense_off : kb * 1024 + lane * 16;
      const int32_t o1 = is_dense ? o0 + 256 : 0x40000000;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        st.v0[g][sl] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ar, sl * slab_bytes + o0, 0, 0));
        st.v1[g][sl] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ar, sl * slab_bytes + o1, 0, 0));
        st.m[g][sl] = __builtin_amdgcn_raw_buffer_load_b32(mr, (sl * 2 * B2 + lane * (B2 / 32) + kb * 2) & ~3, 0, 0);
      }
    }
    const int32_t col = live ? (s0 + it) * 128 + q * 16 : 0x40000000;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int32_t row = (mb * 16 + r) * int32_t(d.ldx) * 2;
      st.b[mb][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, row + col, 0, 0));
      st.b[mb][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, row + col + 64, 0, 0));
    }
  };

  f32x4_t acc[RG][4][MB];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j) acc[g][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Every slab runs on v_smfmac: the first pass for both kinds (a sparse
  // chunk with its index word, or positions 0,1 of every group of a dense
  // piece, index 0x4444), the second pass for dense slabs (positions 2,3,
  // index 0xEEEE).  The selects are bit-selects on an opaque mask so they
  // stay branch-free.
  auto compute = [&](const GemmRxStage<MB, RG>& st, int32_t it) {
    const int mshift = ((lane * (B2 / 32) + ((s0 + it) % kStepsPerTile) * 2) & 2) * 8;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int32_t ti = st.ti[g];
      if (ti == kNone) continue;
      const bool is_dense = ti >= 0;
      uint32_t dm = is_dense ? ~0u : 0u;
      asm("" : "+v"(dm));
      uint4 a0[4], a1[4];
      uint32_t i0[4];
      if constexpr (META == HYB_META_MASK8) {
        // 4:8: a sparse slab's sixteen columns per lane, expanded, take the
        // place of the dense slab's two chunk pieces; both kinds run both
        // passes.
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const u32x4_t v0 = st.v0[g][sl], v1 = st.v1[g][sl];
          uint32_t e[8];
          expand8_lane(lut8, v0[0], v0[1], v0[2], v0[3], (st.m[g][sl] >> mshift) & 0xFFFFu, e);
          const uint32_t l0 = bitsel(dm, v0[0], e[0]), l1 = bitsel(dm, v0[1], e[1]);
          const uint32_t l2 = bitsel(dm, v0[2], e[2]), l3 = bitsel(dm, v0[3], e[3]);
          const uint32_t h0 = bitsel(dm, v1[0], e[4]), h1 = bitsel(dm, v1[1], e[5]);
          const uint32_t h2 = bitsel(dm, v1[2], e[6]), h3 = bitsel(dm, v1[3], e[7]);
          a0[sl] = make_uint4(l0, l2, h0, h2);
          a1[sl] = make_uint4(l1, l3, h1, h3);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
            acc[g][sl][mb] = smfmac16x16x64<DT>(a0[sl], st.b[mb][0], st.b[mb][1], 0x4444u, acc[g][sl][mb]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
            acc[g][sl][mb] = smfmac16x16x64<DT>(a1[sl], st.b[mb][0], st.b[mb][1], 0xEEEEu, acc[g][sl][mb]);
        continue;
      }
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const u32x4_t v0 = st.v0[g][sl], v1 = st.v1[g][sl];
        a0[sl] = make_uint4(v0[0], bitsel(dm, v0[2], v0[1]), bitsel(dm, v1[0], v0[2]), bitsel(dm, v1[2], v0[3]));
        u32x4_t t = {v0[1], v0[3], v1[1], v1[3]};
        asm("" : "+v"(t));
        a1[sl] = __builtin_bit_cast(uint4, t);
        i0[sl] = bitsel(dm, 0x4444u, idx2_word<META>((st.m[g][sl] >> mshift) & 0xFFFFu));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          acc[g][sl][mb] = smfmac16x16x64<DT>(a0[sl], st.b[mb][0], st.b[mb][1], i0[sl], acc[g][sl][mb]);
      if (is_dense) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
            acc[g][sl][mb] = smfmac16x16x64<DT>(a1[sl], st.b[mb][0], st.b[mb][1], 0xEEEEu, acc[g][sl][mb]);
      }
    }
  };

  // STAGES-deep ring, unrolled so every stage index is a compile-time
  // constant; loads of the next STAGES-1 steps are in flight while a step
  // is multiplied.
  GemmRxStage<MB, RG> st[STAGES];
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) load(st[s], s);
  for (int32_t i = 0; i < cnt; i += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      load(st[(s + STAGES - 1) % STAGES], i + s + STAGES - 1);
      if (i + s < cnt) compute(st[s], i + s);
    }
  }

  // Low-rank term: token block mb by wavefront mb % WAVES, into that
  // wavefront's partial sums (the tree below keeps a fixed order).
  if (d.rank > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb % WAVES != wave) continue;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        if (n0 + 64 * g >= d.n) continue;
        f32x4_t c[4][1] = {{acc[g][0][mb]}, {acc[g][1][mb]}, {acc[g][2][mb]}, {acc[g][3][mb]}};
        lr_block<DT, 4, 1>(c, d, n0 + 64 * g, m0 + 16 * mb, lane);
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) acc[g][sl][mb] = c[sl][0];
      }
    }
  }

  // Tree reduction: wavefronts w >= h hand their sums to w - h, for
  // h = WAVES/2, ..., 1.
#pragma unroll
  for (int h = WAVES / 2; h >= 1; h /= 2) {
    if (wave >= h && wave < 2 * h) {
      float* dst = red[wave - h];
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            *reinterpret_cast<f32x4_t*>(dst + (((g * 4 + sl) * MB + mb) * 64 + lane) * 4) = acc[g][sl][mb];
    }
    __syncthreads();
    if (wave < h) {
      const float* src = red[wave];
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[g][sl][mb] += *reinterpret_cast<const f32x4_t*>(src + (((g * 4 + sl) * MB + mb) * 64 + lane) * 4);
    }
    __syncthreads();
  }
  if (wave != 0) return;

  // acc[g][sl][mb] lane L holds rows n0 + 64 g + 16 sl + 4 (L/16) + 0..3 of
  // token m0 + 16 mb + L%16.
  const bool vec_ok = (d.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = int64_t(m0) + mb * 16 + r;
    if (m >= d.m) continue;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      if (n0 + 64 * g >= d.n) continue;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int64_t n = int64_t(n0) + 64 * g + sl * 16 + q * 4;
        const f32x4_t v = acc[g][sl][mb];
        const int64_t base = m * d.ldy + n;
        if (d.ydt == HYB_F32) {
          float* dst = static_cast<float*>(y) + base;
          if (vec_ok) {
            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = v[e];
          }
        } else {
          uint16_t* dst = static_cast<uint16_t*>(y) + base;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = d.ydt == HYB_BF16 ? round16<HYB_BF16>(v[e]) : round16<HYB_F16>(v[e]);
        }
      }
    }
  }
}

// ------------------------------------------------------------ GEMM (LDS) --
//
// Large-M variant: a workgroup covers 256 weight rows (four 64-row groups)
// and BM = 16 * MB tokens.  With four wavefronts each owns a row group and
// all BM tokens; with eight, two wavefronts share a row group and split the
// tokens.  Every K step (64 columns) the workgroup streams its weight pieces
// (8 x 1 KiB per row group: two chunks per slab, the second an empty
// out-of-range read for a sparse slab), the slabs' metadata words and the X
// tile (BM rows x 128 B) straight into LDS with buffer-load-to-LDS
// instructions, STAGES - 1 steps ahead, so the pipeline depth costs no
// registers.  The loads are issued from inline assembly: the compiler then
// does not tie every LDS read to every DMA in flight (which would drain the
// pipeline each step), and the waits are explicit -- every wavefront issues
// the same number of loads per step, so "at most (STAGES-2) steps of loads
// outstanding" followed by a workgroup barrier marks a step's LDS data
// complete and visible.  The X tile's 16-byte slots are XOR-swizzled by
// (row >> 1) & 7 so the B-operand reads of 16 rows hit distinct banks.
typedef __attribute__((ext_vector_type(4))) int srd_t;

__device__ __forceinline__ srd_t make_srd(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return srd_t{__builtin_amdgcn_readfirstlane(int(a & 0xFFFFFFFFu)),
               __builtin_amdgcn_readfirstlane(int((a >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane(int(bytes)), kBufDword3};
}

// 16 bytes per lane from srd + voffset into LDS at lds + 16 * lane.
template <bool NT>
__device__ __forceinline__ void dma16(srd_t srd, uint32_t lds, int voffset) {
  if constexpr (NT) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(lds), "v"(voffset), "s"(srd) : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voffset), "s"(srd) : "memory", "m0");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  // generic -> LDS address space, then the 32-bit LDS offset
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Workgroups are dispatched round-robin over the 8 XCDs (linear id L runs
// on XCD L % 8), each XCD with its own L2.  The launch is a 1-D grid; XCD x
// takes a contiguous range of a grouped order in which kGroupN consecutive
// row blocks are swept across all token blocks before the next group, so the
// workgroups that run together on one XCD share both their weight rows and
// their X tiles in that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroupN = HYB_GEMM_GROUP_N;

__device__ __forceinline__ void xcd_grouped_block(int32_t gx, int32_t& nb, int32_t& mb) {
  const int32_t total = int32_t(gridDim.x);  // gx row blocks x gy token blocks
  const int32_t gy = total / gx;
  const int32_t L = int32_t(blockIdx.x);
  const int32_t xcd = L % kXcds, j = L / kXcds;
  const int32_t per = total / kXcds, extra = total % kXcds;
  const int32_t g = xcd * per + (xcd < extra ? xcd : extra) + j;
  const int32_t gn = g / (kGroupN * gy);
  const int32_t first = gn * kGroupN;
  const int32_t width = gx - first < kGroupN ? gx - first : kGroupN;
  const int32_t r = g - first * gy;
  mb = r / width;
  nb = first + r % width;
}

// WAVES = 4: wavefront w owns rows 64w..64w+63 and all BM tokens.
// WAVES = 8: wavefronts w and w+4 share rows 64(w%4).. and split the tokens,
// giving two wavefronts per SIMD so one can multiply while the other waits
// at the barrier or on LDS.  Loads are spread so every wavefront issues the
// same number per step.
template <int B2, int MB, int STAGES, int WAVES>
struct GemmLdsCfg {
  static constexpr int kABytes = 4 * 8 * 1024;               // weight pieces of 4 row groups
  static constexpr int kXBytes = 16 * MB * 128;               // X tile
  static constexpr int kMetaPerGroup = B2 * 8 < 1024 ? 1024 : B2 * 8;
  static constexpr int kMetaBytes = 4 * kMetaPerGroup;
  static constexpr int kStage = kABytes + kXBytes + kMetaBytes;
  // An out-of-range DMA still writes (zeros) to LDS: loads issued only to
  // keep the per-step count constant land in this sink, which nothing reads.
  static constexpr int kSink = 1024;
  static constexpr int kBytes = STAGES * kStage + kSink;
  static constexpr int kSplit = WAVES / 4;                    // wavefronts per row group
  static constexpr int kALoads = 8 / kSplit;                  // weight chunks per wavefront
  static constexpr int kXLoads = kXBytes / 1024 / WAVES;      // X pieces per wavefront
  static constexpr int kMetaLoads = (kMetaPerGroup / 1024 + kSplit - 1) / kSplit;
  static constexpr int kLoadsPerStep = kALoads + kXLoads + kMetaLoads;
  static constexpr int kMBW = MB / kSplit;                    // token blocks per wavefront
};

template <int B2, int DT, int META, int MB, int STAGES, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_lds(const uint4* __restrict__ dense,
                                                  const uint4* __restrict__ val,
                                                  const uint16_t* __restrict__ meta,
                                                  const int32_t* __restrict__ tidx,
                                                  const uint16_t* __restrict__ x,
                                                  void* __restrict__ y, GemmDims d) {
  using Cfg = GemmLdsCfg<B2, MB, STAGES, WAVES>;
  static_assert(Cfg::kXLoads >= 1 && Cfg::kXLoads * WAVES * 1024 == Cfg::kXBytes, "X tile split");
  constexpr int MBW = Cfg::kMBW;
  constexpr int BM = 16 * MB;
  constexpr int kStepsPerTile = B2 / 64;
  extern __shared__ __attribute__((aligned(1024))) char smem_dyn[];
  __shared__ uint4 lut8[META == HYB_META_MASK8 ? 256 : 1];
  // (4:8 only; the first barrier of the main loop precedes every read)
  if constexpr (META == HYB_META_MASK8) fill_expand8_lut(lut8);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % 4;            // row group
  const int wm = wave / 4;            // token half (WAVES = 8)
  const int q = lane >> 4;
  int32_t nb, mbk;
  xcd_grouped_block((d.n + 255) / 256, nb, mbk);
  const int32_t n0 = nb * 256 + wn * 64;
  const int32_t m0 = mbk * BM;
  const bool rows_ok = n0 < d.n;
  const int32_t tn = n0 / d.b1;
  const int rs0 = (n0 - tn * d.b1) / 16;
  const int32_t steps = d.tiles_k * kStepsPerTile;
  const int32_t* __restrict__ trow = tidx + int64_t(tn) * d.tiles_k;
  const int32_t mrows = d.m - m0 < BM ? d.m - m0 : BM;
  const int64_t tile = int64_t(d.b1) * B2;
  const uint32_t smem_base = lds_addr(smem_dyn);

  constexpr int32_t kNone = INT32_MIN;
  auto tile_index = [&](int32_t st) -> int32_t {
    if (!rows_ok || st >= steps) return kNone;
    const int32_t ti = trow[st / kStepsPerTile];
    const bool ok = ti >= 0 ? (ti < d.n_dense) : (~ti < d.n_sparse);
    return ok ? ti : kNone;
  };
  int32_t tis[STAGES];

  // Issue every load of step `st` into stage `sg` (a compile-time index).
  auto issue = [&](int32_t st, int sg, int32_t ti) {
    const uint32_t stage = smem_base + sg * Cfg::kStage;
    const int kb = st % kStepsPerTile;
    const bool live = ti != kNone;
    const bool is_dense = ti >= 0;
    const int32_t slot = is_dense ? ti : ~ti;
    const int32_t slab_bytes = is_dense ? 32 * B2 : 16 * B2;
    const char* base = is_dense
        ? reinterpret_cast<const char*>(dense) + (int64_t(slot) * tile + int64_t(rs0) * 16 * B2) * 2
        : reinterpret_cast<const char*>(val) + (int64_t(slot) * (tile / 2) + int64_t(rs0) * 8 * B2) * 2;
    const srd_t ar = make_srd(live ? base : nullptr, live ? 4 * slab_bytes : 0);
    const int32_t c0 = is_dense ? 2 * kb * 1024 : kb * 1024;
    const int32_t c1 = is_dense ? c0 + 1024 : 0x40000000;
    const uint32_t adst = stage + wn * 8192;
#pragma unroll
    for (int i = 0; i < Cfg::kALoads; ++i) {
      const int c = wm * Cfg::kALoads + i;   // chunk 2*sl + h of this row group
      const int sl = c >> 1;
      const int32_t off = (c & 1) ? c1 : c0;
      dma16<HYB_GEMM_W_NT != 0>(ar, adst + c * 1024, sl * slab_bytes + off + lane * 16);
    }
    // X tile: piece j (8 rows x 128 B); wavefront w loads pieces
    // w * kXLoads ..; lane l -> row 8j + l/8, LDS slot l%8 holding global
    // 16-byte column (l%8) ^ ((row >> 1) & 7).
    const srd_t xr = make_srd(x + int64_t(m0) * d.ldx, st < steps ? uint32_t(mrows * d.ldx * 2) : 0u);
    const uint32_t xdst = stage + Cfg::kABytes;
#pragma unroll
    for (int i = 0; i < Cfg::kXLoads; ++i) {
      const int j = wave * Cfg::kXLoads + i;
      const int row = 8 * j + (lane >> 3);
      const int c8 = (lane & 7) ^ ((row >> 1) & 7);
      dma16<false>(xr, xdst + j * 1024, int(row * d.ldx * 2) + st * 128 + c8 * 16);
    }
    // metadata words of the four slabs (sparse tiles only)
    const char* mbase = reinterpret_cast<const char*>(meta) + (int64_t(slot) * (tile / 16) + int64_t(rs0) * B2) * 2;
    const srd_t mr = make_srd((live && !is_dense) ? mbase : nullptr, (live && !is_dense) ? 8 * B2 : 0);
    const uint32_t mdst = stage + Cfg::kABytes + Cfg::kXBytes + wn * Cfg::kMetaPerGroup;
#pragma unroll
    for (int i = 0; i < Cfg::kMetaLoads; ++i) {
      // piece wm * kMetaLoads + i of the group's metadata (past the end: an
      // empty out-of-range load that keeps the per-step count constant)
      const int piece = wm * Cfg::kMetaLoads + i;
      const bool real = piece < Cfg::kMetaPerGroup / 1024;
      dma16<false>(mr, real ? mdst + piece * 1024 : smem_base + STAGES * Cfg::kStage,
                   real ? piece * 1024 + lane * 16 : 0x40000000);
    }
    tis[sg] = ti;
  };

  f32x4_t acc[4][MBW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Every step runs on v_smfmac with the accumulators updated in place.  A
  // sparse slab is one A operand (its stored chunk) with its index word.  A
  // dense 64-column slab is split into two 2:4 operands: positions 0,1 of
  // every group of four (index word 0x4444) and positions 2,3 (0xEEEE).
  // Lane L (row L%16, lane group g) needs the 16 columns 16g..16g+15, held
  // by lane groups 2(g%2) and 2(g%2)+1 of dense chunk g/2; of the two 16-byte
  // reads, dwords 0 and 2 form the first operand and dwords 1 and 3 the
  // second.  Dense steps thus issue two sparse products per slab, the same
  // matrix-core time as two 16x16x32 MFMAs.
  //
  // Both kinds share the first pass (one product per slab and token block)
  // and its accumulator registers; dense steps add the second pass.  Every
  // LDS read is a whole 16-byte read (the 64 lanes of a read cover 1 KiB
  // without bank conflicts); the weight reads are volatile so the compiler
  // cannot split one into dword reads of the shuffled halves (lanes 16 bytes
  // apart reading single dwords conflict four ways).  A sparse step reads its chunk twice (the second read feeds
  // nothing) so that both kinds run the same instructions up to the second
  // pass.
  auto compute = [&](int sg, int32_t st) {
    const int32_t ti = tis[sg];
    if (ti == kNone) return;
    const char* stage = smem_dyn + sg * Cfg::kStage;
    const char* xsrc = stage + Cfg::kABytes;
    const bool is_dense = ti >= 0;
    const char* wbase = stage + wn * 8192;
    const int r_off = is_dense ? (q >> 1) * 1024 + ((2 * (q & 1)) * 16 + (lane & 15)) * 16 : lane * 16;
    const int r_off2 = is_dense ? r_off + 256 : r_off;
    const char* msrc = stage + Cfg::kABytes + Cfg::kXBytes + wn * Cfg::kMetaPerGroup +
                       lane * (B2 / 32) + (st % kStepsPerTile) * 2;
    // all-ones for a dense step; opaque to the optimiser so the selects
    // below stay bit-selects instead of becoming branches (each branch would
    // wait for its slab's reads on its own)
    uint32_t dm = is_dense ? ~0u : 0u;
    asm("" : "+v"(dm));
    uint4 a0[4], a1[4];
    uint32_t i0[4];
    if constexpr (META == HYB_META_MASK8) {
      // 4:8: the sparse chunk's two groups per lane, expanded, stand in for
      // the dense slab's two pieces; every step runs both passes.
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const u32x4_t v0 = *(const volatile lds_u32x4_t*)(wbase + (2 * sl) * 1024 + r_off);
        const u32x4_t v1 = *(const volatile lds_u32x4_t*)(wbase + (2 * sl) * 1024 + r_off2);
        const uint32_t m = *reinterpret_cast<const uint16_t*>(msrc + sl * 2 * B2);
        uint32_t e[8];
        expand8_lane(lut8, v0[0], v0[1], v0[2], v0[3], m, e);
        const uint32_t l0 = bitsel(dm, v0[0], e[0]), l1 = bitsel(dm, v0[1], e[1]);
        const uint32_t l2 = bitsel(dm, v0[2], e[2]), l3 = bitsel(dm, v0[3], e[3]);
        const uint32_t h0 = bitsel(dm, v1[0], e[4]), h1 = bitsel(dm, v1[1], e[5]);
        const uint32_t h2 = bitsel(dm, v1[2], e[6]), h3 = bitsel(dm, v1[3], e[7]);
        a0[sl] = make_uint4(l0, l2, h0, h2);
        a1[sl] = make_uint4(l1, l3, h1, h3);
      }
      uint4 bq[MBW][2];
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        const int row = (wm * MBW + mb) * 16 + (lane & 15);
        const int sw = (row >> 1) & 7;
        bq[mb][0] = *reinterpret_cast<const uint4*>(xsrc + row * 128 + ((q ^ sw) * 16));
        bq[mb][1] = *reinterpret_cast<const uint4*>(xsrc + row * 128 + (((q + 4) ^ sw) * 16));
      }
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          acc[sl][mb] = smfmac16x16x64<DT>(a0[sl], bq[mb][0], bq[mb][1], 0x4444u, acc[sl][mb]);
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          acc[sl][mb] = smfmac16x16x64<DT>(a1[sl], bq[mb][0], bq[mb][1], 0xEEEEu, acc[sl][mb]);
      return;
    }
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const u32x4_t v0 = *(const volatile lds_u32x4_t*)(wbase + (2 * sl) * 1024 + r_off);
      const u32x4_t v1 = *(const volatile lds_u32x4_t*)(wbase + (2 * sl) * 1024 + r_off2);
      const uint32_t m = *reinterpret_cast<const uint16_t*>(msrc + sl * 2 * B2);
      a0[sl] = make_uint4(v0[0], bitsel(dm, v0[2], v0[1]), bitsel(dm, v1[0], v0[2]), bitsel(dm, v1[2], v0[3]));
      a1[sl] = make_uint4(v0[1], v0[3], v1[1], v1[3]);
      i0[sl] = bitsel(dm, 0x4444u, idx2_word<META>(m));
    }
    uint4 bq[MBW][2];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      const int row = (wm * MBW + mb) * 16 + (lane & 15);
      const int sw = (row >> 1) & 7;
      bq[mb][0] = *reinterpret_cast<const uint4*>(xsrc + row * 128 + ((q ^ sw) * 16));
      bq[mb][1] = *reinterpret_cast<const uint4*>(xsrc + row * 128 + (((q + 4) ^ sw) * 16));
    }
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        acc[sl][mb] = smfmac16x16x64<DT>(a0[sl], bq[mb][0], bq[mb][1], i0[sl], acc[sl][mb]);
    if (is_dense) {
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          acc[sl][mb] = smfmac16x16x64<DT>(a1[sl], bq[mb][0], bq[mb][1], 0xEEEEu, acc[sl][mb]);
    }
  };

  // Prologue: steps 0 .. STAGES-2.
#pragma unroll
  for (int sg = 0; sg < STAGES - 1; ++sg) issue(sg, sg, tile_index(sg));
  for (int32_t s0 = 0; s0 < steps; s0 += STAGES) {
#pragma unroll
    for (int sg = 0; sg < STAGES; ++sg) {
      const int32_t st = s0 + sg;
      // Step st's loads are complete once at most the STAGES-2 later steps'
      // loads are outstanding; the barrier makes every wavefront's DMA
      // writes visible and frees the stage read in the previous step.
      wait_vmcnt<(STAGES - 2) * Cfg::kLoadsPerStep>();
      __syncthreads();
      constexpr int kAhead = STAGES - 1;
      issue(st + kAhead, (sg + kAhead) % STAGES, tile_index(st + kAhead));
      if (st < steps) compute(sg, st);
    }
  }
  wait_vmcnt<0>();

  if (!rows_ok) return;
  if (d.rank > 0) lr_block<DT, 4, MBW>(acc, d, n0, m0 + wm * MBW * 16, lane);
  const bool vec_ok = (d.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    const int64_t m = int64_t(m0) + (wm * MBW + mb) * 16 + (lane & 15);
    if (m >= d.m) continue;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int64_t n = int64_t(n0) + sl * 16 + q * 4;
      const f32x4_t v = acc[sl][mb];
      const int64_t base = m * d.ldy + n;
      if (d.ydt == HYB_F32) {
        float* dst = static_cast<float*>(y) + base;
        if (vec_ok) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = v[e];
        }
      } else {
        uint16_t* dst = static_cast<uint16_t*>(y) + base;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = d.ydt == HYB_BF16 ? round16<HYB_BF16>(v[e]) : round16<HYB_F16>(v[e]);
      }
    }
  }
}

// ---------------------------------------------------- low-rank project ----
//
// T = X V for the low-rank factor of a sparse + low-rank weight, V held as
// rank rows of k values (row j is column j of V).
//
// Decode sizes (m <= 16): one workgroup per V row and block of MT tokens;
// each thread takes 8-element slices of K at a stride of 8 * 256, two
// products per v_dot2, then the 256 partial sums are reduced across the
// wavefront and, in a fixed order, across the four wavefronts.
template <int DT, int MT>
__global__ __launch_bounds__(256) void k_lr_project(const uint16_t* __restrict__ v, int64_t ldv, int64_t k,
                                                    const uint16_t* __restrict__ x, int32_t m, int64_t ldx,
                                                    float* __restrict__ t, int64_t ldt) {
  __shared__ float part[4][MT];
  const int tid = threadIdx.x;
  const int64_t j = blockIdx.x;
  const int32_t m0 = int32_t(blockIdx.y) * MT;
  const int32_t mc = m - m0 < MT ? m - m0 : MT;
  const uint16_t* vr = v + j * ldv;
  float acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = 0.f;
  for (int64_t kk = int64_t(tid) * 8; kk < k; kk += 256 * 8) {
    const uint4 a = *reinterpret_cast<const uint4*>(vr + kk);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i < mc) {
        const uint4 b = *reinterpret_cast<const uint4*>(x + int64_t(m0 + i) * ldx + kk);
        acc[i] = dot2<DT>(a.x, b.x, acc[i]);
        acc[i] = dot2<DT>(a.y, b.y, acc[i]);
        acc[i] = dot2<DT>(a.z, b.z, acc[i]);
        acc[i] = dot2<DT>(a.w, b.w, acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc[i] += __shfl_xor(acc[i], o, 64);
  }
  if ((tid & 63) == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) part[tid >> 6][i] = acc[i];
  }
  __syncthreads();
  if (tid < mc) t[int64_t(m0 + tid) * ldt + j] = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
}

// Prefill sizes (m > 16): the matrix cores, loading operands straight from
// memory.  One workgroup per 16 tokens and 16 NB ranks (the ranks split
// over at most four workgroups); its eight wavefronts take the 32-column K
// steps round-robin, each holding NB accumulator tiles of 16 ranks.  A operand: V rows (lane L: rank 16 nb + L%16, columns 8 (L/16)
// of the step), B operand: X rows (token L%16), so a tile holds T^T.  The
// wavefronts' sums are added in a fixed tree through LDS.  X is read once
// per workgroup, V once per 16 tokens.
template <int DT, int NB>
__global__ __launch_bounds__(512) void k_lr_project_mfma(const uint16_t* __restrict__ v, int64_t ldv, int32_t rank,
                                                         int64_t k, const uint16_t* __restrict__ x, int32_t m,
                                                         int64_t ldx, float* __restrict__ t, int64_t ldt) {
  constexpr int kWaves = 8;
  __shared__ __attribute__((aligned(16))) float red[kWaves / 2][NB * 4 * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, r = lane & 15;
  const int64_t tok = int64_t(blockIdx.x) * 16 + r;
  const bool tok_ok = tok < m;
  const int32_t jb = int32_t(blockIdx.y) * NB * 16;  // first rank of the workgroup
  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t ksteps = (k + 31) / 32;
#pragma unroll 4
  for (int64_t st = wave; st < ksteps; st += kWaves) {
    const int64_t kk = st * 32 + 8 * q;
    const bool k_ok = kk < k;
    const uint4 bx = (tok_ok && k_ok) ? *reinterpret_cast<const uint4*>(x + tok * ldx + kk) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int32_t j = jb + nb * 16 + r;
      const uint4 av = (j < rank && k_ok) ? *reinterpret_cast<const uint4*>(v + int64_t(j) * ldv + kk)
                                          : make_uint4(0u, 0u, 0u, 0u);
      acc[nb] = mfma16x16x32<DT>(av, bx, acc[nb]);
    }
  }
#pragma unroll
  for (int h = kWaves / 2; h >= 1; h /= 2) {
    if (wave >= h && wave < 2 * h) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f32x4_t*>(&red[wave - h][(nb * 64 + lane) * 4]) = acc[nb];
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] += *reinterpret_cast<const f32x4_t*>(&red[wave][(nb * 64 + lane) * 4]);
    }
    __syncthreads();
  }
  if (wave != 0 || !tok_ok) return;
  // acc[nb] lane L: ranks 16 nb + 4 (L/16) + 0..3 of token L%16
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int32_t j = jb + nb * 16 + 4 * q + e;
      if (j < rank) t[tok * ldt + j] = acc[nb][e];
    }
}

// --------------------------------------------------------- stream read ----
//
// Practical read-rate reference: each wavefront reads four contiguous 1 KiB
// chunks per trip (16 B per lane, non-temporal, like the decode kernel),
// grid-strided over the buffer.
__global__ __launch_bounds__(256) void k_stream_read(const char* __restrict__ p, int64_t bytes,
                                                     uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  constexpr int64_t kSpan = 4 * 1024;
  uint32_t acc = 0;
  for (int64_t base = wave * kSpan; base < bytes; base += nwaves * kSpan) {
    const int32_t n = int32_t(bytes - base < kSpan ? bytes - base : kSpan);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p + base, n);
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, i * 1024 + lane * 16, 0, HYB_W_AUX));
#pragma unroll
    for (int i = 0; i < 4; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

namespace {

template <int DT>
void lr_project_mt(int m, dim3 grid, hipStream_t s, const uint16_t* v, int64_t ldv, int64_t k, const uint16_t* x,
                   int64_t ldx, float* t, int64_t ldt) {
  const dim3 b(256);
  if (m <= 1) hipLaunchKernelGGL((k_lr_project<DT, 1>), grid, b, 0, s, v, ldv, k, x, m, ldx, t, ldt);
  else if (m <= 2) hipLaunchKernelGGL((k_lr_project<DT, 2>), grid, b, 0, s, v, ldv, k, x, m, ldx, t, ldt);
  else if (m <= 4) hipLaunchKernelGGL((k_lr_project<DT, 4>), grid, b, 0, s, v, ldv, k, x, m, ldx, t, ldt);
  else if (m <= 8) hipLaunchKernelGGL((k_lr_project<DT, 8>), grid, b, 0, s, v, ldv, k, x, m, ldx, t, ldt);
  else hipLaunchKernelGGL((k_lr_project<DT, 16>), grid, b, 0, s, v, ldv, k, x, m, ldx, t, ldt);
}

template <int DT>
void lr_project_nb(int nb, dim3 grid, hipStream_t s, const uint16_t* v, int64_t ldv, int rank, int64_t k,
                   const uint16_t* x, int m, int64_t ldx, float* t, int64_t ldt) {
  const dim3 b(512);
  if (nb == 1) hipLaunchKernelGGL((k_lr_project_mfma<DT, 1>), grid, b, 0, s, v, ldv, rank, k, x, m, ldx, t, ldt);
  else if (nb == 2) hipLaunchKernelGGL((k_lr_project_mfma<DT, 2>), grid, b, 0, s, v, ldv, rank, k, x, m, ldx, t, ldt);
  else hipLaunchKernelGGL((k_lr_project_mfma<DT, 4>), grid, b, 0, s, v, ldv, rank, k, x, m, ldx, t, ldt);
}

}  // namespace

hipError_t launch_lr_project(const void* v, int64_t ldv, int rank, int64_t k, int dtype, const void* x, int m,
                             int64_t ldx, float* t, int64_t ldt, hipStream_t s) {
  const auto* vv = static_cast<const uint16_t*>(v);
  const auto* xx = static_cast<const uint16_t*>(x);
  if (m <= 16) {
    const int mt = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : m <= 8 ? 8 : 16;
    const dim3 grid(static_cast<unsigned>(rank), static_cast<unsigned>((m + mt - 1) / mt));
    if (dtype == HYB_BF16) lr_project_mt<HYB_BF16>(m, grid, s, vv, ldv, k, xx, ldx, t, ldt);
    else lr_project_mt<HYB_F16>(m, grid, s, vv, ldv, k, xx, ldx, t, ldt);
  } else {
    const int blocks = (rank + 15) / 16;  // 16-rank tiles, split over up to four workgroups
    const int nb = blocks <= 4 ? 1 : blocks <= 8 ? 2 : 4;  // tiles per workgroup (a template instance)
    const dim3 grid(static_cast<unsigned>((m + 15) / 16), static_cast<unsigned>((blocks + nb - 1) / nb));
    if (dtype == HYB_BF16) lr_project_nb<HYB_BF16>(nb, grid, s, vv, ldv, rank, k, xx, m, ldx, t, ldt);
    else lr_project_nb<HYB_F16>(nb, grid, s, vv, ldv, rank, k, xx, m, ldx, t, ldt);
  }
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* sink, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, s, static_cast<const char*>(p), bytes, sink);
  return hipGetLastError();
}

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

int device_cus();

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

struct GemvPtrs {
  const uint4* dense;
  const uint4* val;
  const uint16_t* meta;
  const int32_t* tidx;
  const uint16_t* x;
  void* y;
};

template <int MT, int DT, int META, bool LR, int W>
void gemv_b2(int b2, dim3 grid, hipStream_t s, const GemvPtrs& q, const GemvDims& d) {
  const dim3 block(64 * W);
  switch (b2) {
    case 64:
      hipLaunchKernelGGL((k_gemv<MT, 64, DT, META, W, kGemvStages, LR>), grid, block, 0, s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d);
      break;
    case 128:
      hipLaunchKernelGGL((k_gemv<MT, 128, DT, META, W, kGemvStages, LR>), grid, block, 0, s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d);
      break;
    default:
      hipLaunchKernelGGL((k_gemv<MT, 256, DT, META, W, kGemvStages, LR>), grid, block, 0, s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d);
      break;
  }
}

// MT-token variant with the wavefront count of gemv_waves.
template <int MT, int DT, int META, bool LR>
void gemv_w(int waves, int b2, dim3 grid, hipStream_t s, const GemvPtrs& q, const GemvDims& d) {
  if constexpr (MT <= 4) {
    if (waves == 8) return gemv_b2<MT, DT, META, LR, 8>(b2, grid, s, q, d);
  } else {
    if (waves == 16) return gemv_b2<MT, DT, META, LR, 16>(b2, grid, s, q, d);
  }
  gemv_b2<MT, DT, META, LR, kGemvWaves>(b2, grid, s, q, d);
}

template <int DT, int META, bool LR>
void gemv_mt(int m, int waves, int b2, dim3 grid, hipStream_t s, const GemvPtrs& q, const GemvDims& d) {
  if (m <= 1) gemv_w<1, DT, META, LR>(waves, b2, grid, s, q, d);
  else if (m <= 2) gemv_w<2, DT, META, LR>(waves, b2, grid, s, q, d);
  else if (m <= 4) gemv_w<4, DT, META, LR>(waves, b2, grid, s, q, d);
  else if (m <= 8) gemv_w<8, DT, META, LR>(waves, b2, grid, s, q, d);
  else gemv_w<16, DT, META, LR>(waves, b2, grid, s, q, d);
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
  const dim3 grid(unsigned(L.n / 16));
  const int w = gemv_waves(L.n / 16, m);
  if (L.dtype == HYB_BF16) {
    if (L.meta == HYB_META_IDX2) gemv_mt<HYB_BF16, HYB_META_IDX2, LR>(m, w, L.b2, grid, s, q, d);
    else if (L.meta == HYB_META_MASK4) gemv_mt<HYB_BF16, HYB_META_MASK4, LR>(m, w, L.b2, grid, s, q, d);
    else gemv_mt<HYB_BF16, HYB_META_MASK8, LR>(m, w, L.b2, grid, s, q, d);
  } else {
    if (L.meta == HYB_META_IDX2) gemv_mt<HYB_F16, HYB_META_IDX2, LR>(m, w, L.b2, grid, s, q, d);
    else if (L.meta == HYB_META_MASK4) gemv_mt<HYB_F16, HYB_META_MASK4, LR>(m, w, L.b2, grid, s, q, d);
    else gemv_mt<HYB_F16, HYB_META_MASK8, LR>(m, w, L.b2, grid, s, q, d);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                       void* y, int y_dtype, int64_t ldy, hipStream_t s) {
  return launch_gemv_impl<false>(L, P, x, m, ldx, y, y_dtype, ldy, nullptr, 0, nullptr, 0, 0, s);
}

bool gemv_preferred(const hyb_layout& L, int m) {
  if (m <= kGemvCrossoverM) return true;
  // 9-16 tokens on a matrix short enough for 16 wavefronts per slab: the
  // decode kernel beats the register-fed product there (1024 and 4096 rows
  // at 16 tokens: 11-12 us against 15-16 us)
  return m <= kMaxGemvM && gemv_waves(L.n / 16, m) == 16;
}

hipError_t launch_gemv_lowrank(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                               const float* t, int64_t ldt, const void* u, int64_t ldu, int rank, void* y,
                               int y_dtype, int64_t ldy, hipStream_t s) {
  return launch_gemv_impl<true>(L, P, x, m, ldx, y, y_dtype, ldy, t, ldt, u, ldu, rank, s);
}

namespace {

template <int MT, int DT, int META, int W>
void gemv_grouped_b2(int b2, dim3 grid, hipStream_t s, const uint16_t* x, const GemvDims& d, const GemvGroup& g) {
  const dim3 block(64 * W);
  switch (b2) {
    case 64:
      hipLaunchKernelGGL((k_gemv_grouped<MT, 64, DT, META, W, kGemvStages>), grid, block, 0, s, x, d, g);
      break;
    case 128:
      hipLaunchKernelGGL((k_gemv_grouped<MT, 128, DT, META, W, kGemvStages>), grid, block, 0, s, x, d, g);
      break;
    default:
      hipLaunchKernelGGL((k_gemv_grouped<MT, 256, DT, META, W, kGemvStages>), grid, block, 0, s, x, d, g);
      break;
  }
}

template <int MT, int DT, int META>
void gemv_grouped_w(int waves, int b2, dim3 grid, hipStream_t s, const uint16_t* x, const GemvDims& d,
                    const GemvGroup& g) {
  if constexpr (MT <= 4) {
    if (waves == 8) return gemv_grouped_b2<MT, DT, META, 8>(b2, grid, s, x, d, g);
  } else {
    if (waves == 16) return gemv_grouped_b2<MT, DT, META, 16>(b2, grid, s, x, d, g);
  }
  gemv_grouped_b2<MT, DT, META, kGemvWaves>(b2, grid, s, x, d, g);
}

template <int DT, int META>
void gemv_grouped_mt(int m, int waves, int b2, dim3 grid, hipStream_t s, const uint16_t* x, const GemvDims& d,
                     const GemvGroup& g) {
  if (m <= 1) gemv_grouped_w<1, DT, META>(waves, b2, grid, s, x, d, g);
  else if (m <= 2) gemv_grouped_w<2, DT, META>(waves, b2, grid, s, x, d, g);
  else if (m <= 4) gemv_grouped_w<4, DT, META>(waves, b2, grid, s, x, d, g);
  else if (m <= 8) gemv_grouped_w<8, DT, META>(waves, b2, grid, s, x, d, g);
  else gemv_grouped_w<16, DT, META>(waves, b2, grid, s, x, d, g);
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
    if (L[0].dtype == HYB_BF16) {
      if (L[0].meta == HYB_META_IDX2) gemv_grouped_mt<HYB_BF16, HYB_META_IDX2>(m, w, L[0].b2, grid, s, xp, d, g);
      else if (L[0].meta == HYB_META_MASK4) gemv_grouped_mt<HYB_BF16, HYB_META_MASK4>(m, w, L[0].b2, grid, s, xp, d, g);
      else gemv_grouped_mt<HYB_BF16, HYB_META_MASK8>(m, w, L[0].b2, grid, s, xp, d, g);
    } else {
      if (L[0].meta == HYB_META_IDX2) gemv_grouped_mt<HYB_F16, HYB_META_IDX2>(m, w, L[0].b2, grid, s, xp, d, g);
      else if (L[0].meta == HYB_META_MASK4) gemv_grouped_mt<HYB_F16, HYB_META_MASK4>(m, w, L[0].b2, grid, s, xp, d, g);
      else gemv_grouped_mt<HYB_F16, HYB_META_MASK8>(m, w, L[0].b2, grid, s, xp, d, g);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
  auto rx_wgs = [&](int i) {
    return ((groups + kShapes[i][2] - 1) / kShapes[i][2]) * ((m + 16 * kShapes[i][0] - 1) / (16 * kShapes[i][0]));
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
    if (best == 4 && best_rounds >= 2 && ((n + 255) / 256) * ((m + 63) / 64) <= cus)
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
    if ((m + 16 * kShapes[i][0] - 1) / (16 * kShapes[i][0]) > 65535) continue;
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

namespace {

template <int B2, int DT, int META, int MB, int STAGES, int WAVES>
hipError_t gemm_lds_go(const hyb_layout& L, const GemvPtrs& q, int m, const GemmDims& d, hipStream_t s) {
  using Cfg = GemmLdsCfg<B2, MB, STAGES, WAVES>;
  static_assert(Cfg::kBytes <= 160 * 1024, "LDS budget");
  const int64_t gm = (int64_t(m) + 16 * MB - 1) / (16 * MB);
  const int64_t gn = (L.n + 255) / 256;
  if (gn * gm >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
  // 1-D launch of gn * gm workgroups, mapped to (row block, token block)
  // inside the kernel.
  hipLaunchKernelGGL((k_gemm_lds<B2, DT, META, MB, STAGES, WAVES>), dim3(unsigned(gn * gm)), dim3(64 * WAVES),
                     size_t(Cfg::kBytes), s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d);
  return hipGetLastError();
}

template <int B2, int DT, int META, int MB, int WAVES, int STAGES, int RG = 1>
hipError_t gemm_rx_go(const hyb_layout& L, const GemvPtrs& q, int m, const GemmDims& d, hipStream_t s) {
  const int64_t gm = (int64_t(m) + 16 * MB - 1) / (16 * MB);
  if (gm > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid(unsigned((L.n + 64 * RG - 1) / (64 * RG)), unsigned(gm));
  hipLaunchKernelGGL((k_gemm_rx<B2, DT, META, MB, WAVES, STAGES, RG>), grid, dim3(64 * WAVES), 0, s, q.dense,
                     q.val, q.meta, q.tidx, q.x, q.y, d);
  return hipGetLastError();
}

// Three LDS stages where they fit (with the 4 KiB selector table of 4:8
// tiles), else two.
template <int B2, int MB, int WAVES, int META>
constexpr int lds_stages() {
  return GemmLdsCfg<B2, MB, 3, WAVES>::kBytes + (META == HYB_META_MASK8 ? 4096 : 0) <= 160 * 1024 ? 3 : 2;
}

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

template <int B2, int DT, int META>
hipError_t gemm_shape(const hyb_layout& L, const GemvPtrs& q, int m, const GemmDims& d, hipStream_t s) {
  const GemmRoute r = gemm_route(L.n, m, device_cus());
  if (r.kernel == kRouteLds) {
    switch (r.mb) {
      case 16: return gemm_lds_go<B2, DT, META, 16, lds_stages<B2, 16, 8, META>(), 8>(L, q, m, d, s);
      case 12: return gemm_lds_go<B2, DT, META, 12, lds_stages<B2, 12, 8, META>(), 8>(L, q, m, d, s);
      case 8: return gemm_lds_go<B2, DT, META, 8, lds_stages<B2, 8, 8, META>(), 8>(L, q, m, d, s);
      default: return gemm_lds_go<B2, DT, META, 4, lds_stages<B2, 4, 8, META>(), 8>(L, q, m, d, s);
    }
  }
  if (r.rg == 2) {
    if (r.mb == 2) return gemm_rx_go<B2, DT, META, 2, 4, 2, 2>(L, q, m, d, s);
    return gemm_rx_go<B2, DT, META, 4, 4, 2, 2>(L, q, m, d, s);
  }
  switch (r.mb) {
    case 1:
      if (r.waves == 8) return gemm_rx_go<B2, DT, META, 1, 8, 2>(L, q, m, d, s);
      return gemm_rx_go<B2, DT, META, 1, 4, 2>(L, q, m, d, s);
    case 2: return gemm_rx_go<B2, DT, META, 2, 8, 2>(L, q, m, d, s);
    default: return gemm_rx_go<B2, DT, META, 4, 8, 2>(L, q, m, d, s);
  }
}

template <int DT, int META>
hipError_t gemm_b2(const hyb_layout& L, const GemvPtrs& q, int m, const GemmDims& d, hipStream_t s) {
  switch (L.b2) {
    case 64: return gemm_shape<64, DT, META>(L, q, m, d, s);
    case 128: return gemm_shape<128, DT, META>(L, q, m, d, s);
    default: return gemm_shape<256, DT, META>(L, q, m, d, s);
  }
}

}  // namespace

hipError_t launch_gemm(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                       void* y, int y_dtype, int64_t ldy, hipStream_t s, const float* t, int64_t ldt,
                       const void* u, int64_t ldu, int rank) {
  GemvPtrs q{static_cast<const uint4*>(P.dense), static_cast<const uint4*>(P.val),
             static_cast<const uint16_t*>(P.meta), P.tidx, static_cast<const uint16_t*>(x), y};
  GemmDims d{};
  d.ldx = ldx;
  d.ldy = ldy;
  d.n = int32_t(L.n);
  d.m = m;
  d.tiles_k = int32_t(L.tiles_k);
  d.n_dense = int32_t(L.n_dense);
  d.n_sparse = int32_t(L.n_sparse);
  d.b1 = L.b1;
  d.ydt = y_dtype;
  d.t = t;
  d.u = static_cast<const uint16_t*>(u);
  d.ldt = ldt;
  d.ldu = ldu;
  d.rank = rank;
  if (L.dtype == HYB_BF16) {
    if (L.meta == HYB_META_IDX2) return gemm_b2<HYB_BF16, HYB_META_IDX2>(L, q, m, d, s);
    if (L.meta == HYB_META_MASK4) return gemm_b2<HYB_BF16, HYB_META_MASK4>(L, q, m, d, s);
    return gemm_b2<HYB_BF16, HYB_META_MASK8>(L, q, m, d, s);
  }
  if (L.meta == HYB_META_IDX2) return gemm_b2<HYB_F16, HYB_META_IDX2>(L, q, m, d, s);
  if (L.meta == HYB_META_MASK4) return gemm_b2<HYB_F16, HYB_META_MASK4>(L, q, m, d, s);
  return gemm_b2<HYB_F16, HYB_META_MASK8>(L, q, m, d, s);
}

}  // namespace hyb
