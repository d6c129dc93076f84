// Internal interface between the host-side argument checks (hyb_api.cpp) and
// the kernel launchers (hyb_pack.hip, hyb_gemv.hip, hyb_gemm.hip, hyb_lowrank.hip).  Everything reaching a launcher has
// already been validated.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/hyb.h"

namespace hyb {

// Wavefronts per 16-row slab of the decode kernel on matrices with at least
// two slabs per compute unit (chosen by measurement; see gemv_waves).
#ifndef HYB_GEMV_WAVES
#define HYB_GEMV_WAVES 4
#endif
constexpr int kGemvWaves = HYB_GEMV_WAVES;
// Decode kernel handles up to this many tokens per launch.
constexpr int kMaxGemvM = 16;
// hyb_gemm runs the decode kernel up to this many tokens on every matrix
// (it is the faster kernel there, up to 1.9x); from 5 tokens the decode
// kernel's cost steps up (14336 x 4096: 17.7 us at 4 tokens, 22 at 5) and
// the matrix cores take the product except on short matrices
// (gemv_preferred).
constexpr int kGemvCrossoverM = 4;
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
// Whether hyb_gemm should run m tokens on the decode kernel (m <= 4, or
// m <= 16 on a matrix of at most one 16-row slab per compute unit).
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
// Compute units of the current device (256 when no device is visible);
// cached per device.
int device_cus();
// Wavefronts per 16-row slab of the decode kernel for a matrix of `slabs`
// slabs at m tokens.
int gemv_waves(int64_t slabs, int m);
// Slabs the decode kernel runs whole when it cuts the last round's slabs
// into 8-row halves (all `slabs` where it does not); the launch takes
// full + 2 (slabs - full) workgroups.
int64_t gemv_full_slabs(int64_t slabs, int cus);
// Kernel and workgroup shape of a product (hyb_gemm_shape).
constexpr int kRouteDecode = 1;    // k_gemv
constexpr int kRouteRegister = 2;  // k_gemm_rx
constexpr int kRouteLds = 3;       // k_gemm_lds
constexpr int kRouteSplit = 4;     // k_gemm_split or k_gemm_lds_split (rg 4), then its sum kernel
struct GemmRoute {
  int kernel;  // kRoute*
  int mb;      // token blocks of 16 per workgroup (0: the decode kernel)
  int waves;   // wavefronts per workgroup
  int rg;      // 64-row groups per workgroup (0: the decode kernel's 16-row slabs;
               // 4: the LDS-fed kernel, also when split)
  int groups;  // workgroups of a split launch (0 otherwise)
  int rows0;   // 192- and 256-token tiles cut into K parts: the first rows0
               // 256-row blocks run whole in a plain launch first, the K
               // parts cover the blocks after them (0: all blocks in parts)
};
// A split launch runs one workgroup per CU on at most this many CUs (its
// workgroups hold partial sums in a workspace of at most kSplitMaxBytes) ...
constexpr int64_t kSplitMaxCus = 256;
// ... and gives each wavefront at least this many K steps.
constexpr int64_t kSplitMinSteps = 2;
// Largest split_workspace_bytes of any route: 256 workgroups x 2 pieces x
// (256 rows x 128 tokens x 4 bytes), the LDS-fed 128-token shape.
constexpr size_t kSplitMaxBytes = size_t(kSplitMaxCus) * 2 * 4 * 8 * 4096;
// What the matrix-core kernels run for m >= 1 tokens on an n x k matrix
// over `cus` compute units.
GemmRoute gemm_route(int64_t n, int64_t k, int m, int64_t cus);
GemmRoute gemm_route(const hyb_layout& L, int m, int64_t cus);
// Workspace bytes of a route (nonzero only for a split launch).
size_t split_workspace_bytes(const GemmRoute& r);
// What hyb_gemm runs on the current device (decode kernel included).
GemmRoute gemm_route_device(const hyb_layout& L, int m);
// Device address, on the current device, of the library's static scratch
// array of kSplitMaxBytes (looked up once per device; no allocation).
hipError_t split_scratch(void** out);
// With rank > 0 the kernels add T U^T (t: m x rank fp32, u: n x rank) to
// every output before it is stored.  A split route runs split when `ws`
// holds at least split_workspace_bytes of it (device memory, 16-byte
// aligned, no initial contents needed), else as the same shape unsplit.
hipError_t launch_gemm(const hyb_layout& L, const hyb_packed& P, const void* x, int m,
                       int64_t ldx, void* y, int y_dtype, int64_t ldy, hipStream_t s, void* ws,
                       size_t ws_bytes, const float* t = nullptr, int64_t ldt = 0, const void* u = nullptr,
                       int64_t ldu = 0, int rank = 0);

}  // namespace hyb
