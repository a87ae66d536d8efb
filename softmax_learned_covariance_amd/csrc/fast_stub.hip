// Placeholder for the bf16 MFMA fast path: reports "not supported" so every call
// takes the generic kernels.
#include "plx_internal.h"

namespace plx {
bool fast_fwd_supported(const Geom&) { return false; }
size_t fast_fwd_workspace(const Geom&) { return 0; }
hipError_t launch_fast_fwd(const Geom&, const void*, const void*, const void*, const void*, float*,
                           float*, float*, float*, int, void*, hipStream_t) {
  return hipErrorNotSupported;
}
bool fast_bwd_supported(const Geom&) { return false; }
size_t fast_bwd_workspace(const Geom&) { return 0; }
hipError_t launch_fast_bwd(const Geom&, const void*, const void*, const void*, const void*,
                           const float*, const void*, const float*, const float*, const float*,
                           float*, float*, float*, float*, int, void*, hipStream_t) {
  return hipErrorNotSupported;
}
bool fast_decode_supported(const Geom&) { return false; }
size_t fast_decode_workspace(const Geom&) { return 0; }
hipError_t launch_fast_decode(const Geom&, const void*, const void*, const void*, const int32_t*,
                              const void*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace plx
