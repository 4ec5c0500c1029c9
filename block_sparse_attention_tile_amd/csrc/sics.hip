#include "vsa_internal.h"
namespace vsa {
hipError_t launch_sics(const Geo&, const Ws&, const uint16_t*, const uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace vsa
