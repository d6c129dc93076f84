// Device-side helpers shared by the kernel translation units of libhyb
// (gfx950, MI355X): vector types, 16-bit widening and rounding, dot
// products, 2:4 and 4:8 metadata decoding, buffer resources, and the
// argument structs of the products.  The definitions sit in an unnamed
// namespace, so each translation unit has its own copy.
//
// Stream format (include/hyb.h): every 1 KiB of the dense or value stream is
// a piece of one 16-row slab of one tile, and lane L (0..63) of a wavefront
// owns 16 bytes of it:
//   dense chunk  = 16 rows x 32 columns; lane L: row L%16, columns 8*(L/16)..+7
//   value chunk  = 16 rows x 64 columns (32 stored values per row); lane L:
//                  row L%16, the four groups 4*(L/16)..+3, two values each
//   metadata     = one 16-bit word per (value chunk, lane), a lane's words
//                  for the b2/64 chunks of a slab back to back.
// A wavefront therefore streams each slab with fully coalesced 16-byte loads,
// and the dense chunk is also the A-operand layout of the 16x16x32 MFMA.
#ifndef HYB_DEVICE_H_
#define HYB_DEVICE_H_

#include <hip/hip_runtime.h>

#include <cstdint>

#include "hyb_internal.h"

// Tuning knobs of the decode kernel (defaults chosen by measurement):
// wavefronts per workgroup splitting a slab's tile columns, tiles kept in
// flight per wavefront, and the cache-policy bits of the weight loads.
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
#ifndef HYB_W_AUX
#define HYB_W_AUX 2  // non-temporal: the weights are read once per product
#endif
// The decode kernel's metadata and x loads: non-temporal as well (the
// metadata is read once; measured 0.4 us faster on the 8B up projection).
#ifndef HYB_M_AUX
#define HYB_M_AUX 2
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

// v_perm selector that gathers the 16-bit elements i0 and i1 (each 0..3) of
// the 64-bit pair {hi:lo} into one dword (i0 in the low half): bytes
// 2 i0, 2 i0 + 1, 2 i1, 2 i1 + 1.  (i0 | i1 << 16) * 0x202 places 2 i0 and
// 2 i1 in bytes 0 and 2 and their copies in bytes 1 and 3 (a 24-bit product).
__device__ __forceinline__ uint32_t gather_selector(uint32_t i0, uint32_t i1) {
  return (i0 | (i1 << 16)) * 0x202u + 0x01000100u;
}

// The four gather selectors of one 16-bit metadata word (groups g = 0..3 at
// bits 4g..4g+3).  For idx2 codes (i0 | i1 << 2) the fields are moved in
// place for all four groups at once: c holds i0 of group g at bit 4g and i1
// at bit 16 + 4g.
template <int META>
__device__ __forceinline__ void word_selectors(uint32_t word, uint32_t (&sel)[4]) {
  if constexpr (META == HYB_META_IDX2) {
    const uint32_t c = (word & 0x3333u) | ((word << 14) & 0x33330000u);
#pragma unroll
    for (int g = 0; g < 4; ++g) sel[g] = ((c >> (4 * g)) & 0x30003u) * 0x202u + 0x01000100u;
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t i0, i1;
      nibble_positions_t<META>((word >> (4 * g)) & 0xFu, i0, i1);
      sel[g] = gather_selector(i0, i1);
    }
  }
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

// Device addresses of one product's operands.
struct GemvPtrs {
  const uint4* dense;
  const uint4* val;
  const uint16_t* meta;
  const int32_t* tidx;
  const uint16_t* x;
  void* y;
};

constexpr int kGemvStages = HYB_GEMV_STAGES;

}  // namespace
}  // namespace hyb

#endif  // HYB_DEVICE_H_
