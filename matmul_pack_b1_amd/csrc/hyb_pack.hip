// Pack and unpack kernels of libhyb (gfx950): dense tiles copied, 2:4 and
// 4:8 sparse tiles pruned by magnitude and compressed to values plus
// metadata, and the inverse.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hyb_device.h"

namespace hyb {
namespace {

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

}  // namespace hyb
