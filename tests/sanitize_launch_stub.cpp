// Test infrastructure: stand-ins for libhyb's kernel launchers, so that the
// host-side files (argument checks, planning, routing) can be built by the
// host compiler alone with the address and undefined-behaviour sanitizers.
// Every launcher reports hipErrorNoDevice -- what a launch returns on a
// machine without a GPU -- so calls that pass validation end in
// HYB_ERR_HIP exactly as they do against the real library there.
#include "../matmul_pack_b1_amd/csrc/hyb_internal.h"

namespace hyb {

hipError_t launch_pack(const hyb_layout&, const void*, int64_t, const hyb_packed&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_unpack(const hyb_layout&, const hyb_packed&, void*, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gemv(const hyb_layout&, const hyb_packed&, const void*, int, int64_t, void*, int, int64_t,
                       hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_lr_project(const void*, int64_t, int, int64_t, int, const void*, int, int64_t, float*, int64_t,
                             hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gemv_lowrank(const hyb_layout&, const hyb_packed&, const void*, int, int64_t, const float*,
                               int64_t, const void*, int64_t, int, void*, int, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gemv_grouped(int, const hyb_layout*, const hyb_packed*, const void*, int, int64_t, void* const*,
                               int, const int64_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_stream_read(const void*, int64_t, uint32_t*, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t split_scratch(void**) { return hipErrorNoDevice; }
hipError_t launch_gemm(const hyb_layout&, const hyb_packed&, const void*, int, int64_t, void*, int, int64_t,
                       hipStream_t, void*, size_t, const float*, int64_t, const void*, int64_t, int) {
  return hipErrorNoDevice;
}

}  // namespace hyb
