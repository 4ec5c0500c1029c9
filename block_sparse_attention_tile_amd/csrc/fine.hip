#include "vsa_internal.h"
namespace vsa {
hipError_t launch_fine_select(const Geo&, const Ws&, const uint16_t*, const uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_fine_attend(const Geo&, const Ws&, const uint16_t*, const uint16_t*,
                              const uint16_t*, uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace vsa
