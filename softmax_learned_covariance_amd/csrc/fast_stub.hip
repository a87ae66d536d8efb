// The fast decode is not written yet: report "not supported" so the
// generic kernels serve those calls.
#include "plx_internal.h"

namespace plx {
bool fast_decode_supported(const Geom&) { return false; }
size_t fast_decode_workspace(const Geom&) { return 0; }
hipError_t launch_fast_decode(const Geom&, const void*, const void*, const void*, const int32_t*,
                              const void*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace plx
