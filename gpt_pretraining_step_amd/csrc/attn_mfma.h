// MFMA flash attention for head_dim 128 on gfx950 (declarations).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {
bool attn_mfma_supported(int T, int H, int Hkv, int hd);
bool attn_mfma_bwd_supported(int T, int H, int Hkv, int hd);
// score_bound > 0: every |q . k| / sqrt(hd) is at most score_bound (the
// caller's guarantee; 0 = unknown)
hipError_t attn_mfma_fwd(const void* qkv, void* o, float* lse, int B, int T, int H, int Hkv,
                         int hd, int W, hipStream_t s, float score_bound);
size_t attn_mfma_bwd_scratch_bytes(int B, int T, int H, int hd);
// nrq / nrk / ncs (all or none): 1/rms of the rotated q and k heads and the
// (cos, sin) table; given, the dq and dk written are the gradients w.r.t.
// the raw q and k (RoPE-then-QK-norm backward fused into the epilogues)
// s2 (optional, with fork / join events): the dQ pass runs there, beside
// the dK pass on s, and the dV pass on s4 (with join4) or after dQ on s2
// (the three passes are independent once Delta is formed); s waits for
// them before returning
hipError_t attn_mfma_bwd(const void* qkv, const void* o, const float* lse, const void* dout,
                         void* dqkv, float* delta, void* scratch, int B, int T, int H, int Hkv,
                         int hd, int W, hipStream_t s, const float* nrq, const float* nrk,
                         const float* ncs, hipStream_t s2 = nullptr, hipEvent_t fork = nullptr,
                         hipEvent_t join = nullptr, hipStream_t s4 = nullptr,
                         hipEvent_t join4 = nullptr);
}  // namespace gk
