// Internal interface between the host-side argument checks (hyb_api.cpp) and
// the kernel launchers (hyb_kernels.hip).  Everything reaching a launcher has
// already been validated.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/hyb.h"

namespace hyb {

// Decode kernel handles up to this many tokens per launch.
constexpr int kMaxGemvM = 16;
// hyb_gemm runs the decode kernel up to this many tokens and the
// matrix-core kernels above (measured: from 9 tokens the register-fed
// matrix-core kernel is 1.4-1.9x faster on every workload shape; up to 4
// the decode kernel is faster; between they are even).
constexpr int kGemvCrossoverM = 8;
// Matrices per grouped decode launch (HYB_MAX_GROUP in hyb.h).
constexpr int kMaxGroup = HYB_MAX_GROUP;

hipError_t launch_pack(const hyb_layout& L, const void* w, int64_t ldw, const hyb_packed& P,
                       hipStream_t s);
hipError_t launch_unpack(const hyb_layout& L, const hyb_packed& P, void* w, int64_t ldw,
                         hipStream_t s);
hipError_t launch_gemv(const hyb_layout& L, const hyb_packed& P, const void* x, int m,
                       int64_t ldx, void* y, int y_dtype, int64_t ldy, hipStream_t s);
// Decode product plus the low-rank term T U^T (hyb_gemv_lowrank).
hipError_t launch_lr_project(const void* v, int64_t ldv, int rank, int64_t k, int dtype, const void* x, int m,
                             int64_t ldx, float* t, int64_t ldt, hipStream_t s);
// Whether hyb_gemm should run m tokens on the decode kernel (m <= 8, or
// m <= 16 on a matrix short enough that the decode kernel splits each tile
// row sixteen ways).
bool gemv_preferred(const hyb_layout& L, int m);
hipError_t launch_gemv_lowrank(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                               const float* t, int64_t ldt, const void* u, int64_t ldu, int rank, void* y,
                               int y_dtype, int64_t ldy, hipStream_t s);
// Largest rank of hyb_gemv_lowrank (HYB_MAX_RANK in hyb.h).
constexpr int kMaxRank = HYB_MAX_RANK;
// All matrices share k, b2, dtype and metadata kind (checked by the caller).
hipError_t launch_gemv_grouped(int count, const hyb_layout* L, const hyb_packed* P, const void* x, int m,
                               int64_t ldx, void* const* y, int y_dtype, const int64_t* ldy, hipStream_t s);
hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* sink, int grid, hipStream_t s);
// Kernel and workgroup shape of a product (hyb_gemm_shape).
constexpr int kRouteDecode = 1;    // k_gemv
constexpr int kRouteRegister = 2;  // k_gemm_rx
constexpr int kRouteLds = 3;       // k_gemm_lds
struct GemmRoute {
  int kernel;  // kRoute*
  int mb;      // token blocks of 16 per workgroup (0: the decode kernel)
  int waves;   // wavefronts per workgroup
  int rg;      // 64-row groups per workgroup (0: the decode kernel's 16-row slabs)
};
// What the matrix-core kernels run for m >= 1 tokens on an n-row matrix
// over `cus` compute units.
GemmRoute gemm_route(int64_t n, int m, int64_t cus);
// What hyb_gemm runs on the current device (decode kernel included).
GemmRoute gemm_route_device(const hyb_layout& L, int m);
// With rank > 0 the kernels add T U^T (t: m x rank fp32, u: n x rank) to
// every output before it is stored.
hipError_t launch_gemm(const hyb_layout& L, const hyb_packed& P, const void* x, int m,
                       int64_t ldx, void* y, int y_dtype, int64_t ldy, hipStream_t s,
                       const float* t = nullptr, int64_t ldt = 0, const void* u = nullptr, int64_t ldu = 0,
                       int rank = 0);

}  // namespace hyb
