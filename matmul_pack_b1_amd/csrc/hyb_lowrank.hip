// Low-rank projection kernels of libhyb (gfx950), T = X V for a sparse +
// low-rank weight, and the streaming-read measurement kernel.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hyb_device.h"

namespace hyb {
namespace {

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

}  // namespace hyb
