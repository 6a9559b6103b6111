// MFMA kernels (gfx950) -- placeholder until the matrix-core path lands.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace mla {

bool mfma_absorb_supports(const mla_dims_t&) { return false; }
hipError_t launch_absorb_mfma(const mla_dims_t&, const void*, const void*, const int32_t*, float,
                              const void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
bool mfma_decode_supports(const mla_dims_t&, int64_t, const void*, const void*) { return false; }
hipError_t launch_decode_mfma(const mla_dims_t&, const DecodeArgs&, hipStream_t) {
  return hipErrorNotSupported;
}
bool mfma_out_proj_supports(const mla_dims_t&) { return false; }
hipError_t launch_out_proj_mfma(const mla_dims_t&, const void*, const void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace mla
