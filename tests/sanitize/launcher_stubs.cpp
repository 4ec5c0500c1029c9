// Host-only stand-ins for the kernel launchers of libvsa, so that the host
// code of the C ABI (api.cpp) can be built and run under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  Every launcher
// reports an error; the harness only drives paths that end before a launch.
#include "../../block_sparse_attention_tile_amd/csrc/vsa_internal.h"

namespace vsa {

size_t fine_scratch_bytes(const Geo& g) { return (size_t)g.B * g.H * 4096; }

hipError_t launch_layout(const Geo&, const Ws&, const uint16_t*, const uint16_t*, const uint16_t*, bool,
                         hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_amax(const Geo&, const Ws&, const uint16_t*, const uint16_t*, const uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_untile(const Geo&, const Ws&, int, uint16_t*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_select(const Geo&, const Ws&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attend(const Geo&, const Ws&, const uint16_t*, uint16_t*, hipStream_t, bool) {
  return hipErrorNotSupported;
}
hipError_t launch_sics(const Geo&, const Ws&, const uint16_t*, const uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_profile(const Geo&, const Ws&, const uint16_t*, const uint16_t*, const uint16_t*,
                          hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_fine_select(const Geo&, const Ws&, const uint16_t*, const uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_fine_attend(const Geo&, const Ws&, const uint16_t*, const uint16_t*, const uint16_t*,
                              uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace vsa
