// gla_bwd.hip -- backward kernels of the GLA chunkwise layer for gfx950.
#include "gla_common.h"
#include "gla_internal.h"

namespace gla {

hipError_t launch_chunk_grad(const Plan&, const void*, const void*, const void*, const void*,
                             const float*, const void*, const void*, const void*, void*, void*,
                             void*, float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_rowsum_state(const Plan&, const float*, const float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_dla_carry(const Plan&, const float*, const float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gla
