// bf16 MFMA GEMM for gfx950 (declarations; kernels in k_gemm_mfma.hip).
#pragma once
#include "kernels.h"

namespace gk {
bool mfma_gemm_supported(const GemmDesc& g);
hipError_t mfma_gemm(const GemmDesc& g, hipStream_t s);
size_t mfma_splitk_bytes(int64_t M, int64_t N, int64_t K);
}  // namespace gk
