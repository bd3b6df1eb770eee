// MFMA flash attention for gfx950 (placeholder: the generic kernels serve all shapes).
#include "attn_mfma.h"

namespace gk {
bool attn_mfma_supported(int, int, int, int) { return false; }
hipError_t attn_mfma_fwd(const void*, void*, float*, int, int, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
size_t attn_mfma_bwd_scratch_bytes(int, int, int, int) { return 0; }
hipError_t attn_mfma_bwd(const void*, const void*, const float*, const void*, void*, float*, void*,
                         int, int, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace gk
