// bf16 MFMA GEMM for gfx950 (placeholder: the generic kernel serves all shapes).
#include "gemm_mfma.h"

namespace gk {
bool mfma_gemm_supported(const GemmDesc&) { return false; }
hipError_t mfma_gemm(const GemmDesc&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gk
