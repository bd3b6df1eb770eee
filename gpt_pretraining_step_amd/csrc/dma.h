// Buffer loads straight into LDS (gfx950), shared by the GEMM and attention
// kernels.
//
// buffer_load_dwordx4 ... lds moves 16 bytes per lane from global memory to
// LDS at M0 + 16 * lane: one instruction fills one contiguous 1 KB block, so
// a kernel chooses its LDS layout through the global address each lane
// fetches.  Reads past the descriptor's byte count return zeros.
#pragma once
#include "common.h"

namespace gk {

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// ds_read_b64_tr_b16: in each 16-lane group, lane s points at 4 consecutive
// 16-bit values (row s / 4, columns 4 (s % 4) .. of a 4 x 16 block) and
// receives column s of that block: the 4 values one column holds in the 4
// rows.
__device__ __forceinline__ v4s_t tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)p);
}

static constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, gfx9 family
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t lim = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);   // stride 0
  r[2] = (int)(uint32_t)lim;
  r[3] = kRsrcWord3;
  return r;
}

// One 16-byte-per-lane buffer load into the 1 KB LDS block at `lds` (a wave-
// uniform LDS byte address).  Written as asm so the compiler does not track
// it: the waits for these loads are the explicit vmcnt(0) before each
// barrier of the main loop, and reads of the other stage never wait for them.
// `voff` is the whole byte offset (the scalar offset field stays 0): the
// range check against the descriptor's byte count applies to it.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// One 4-byte-per-lane buffer load into LDS at `lds` + 4 lane: a gather, each
// lane with its own byte offset `voff` (range-checked like dma16's).  Same
// tracking as dma16: waited for by the explicit waits below.
__device__ __forceinline__ void dma4(i32x4_t rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Wait for every buffer-to-LDS load this wave issued (they are not tracked
// by the compiler); follow with a barrier before other waves read the data.
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's vector memory loads are outstanding:
// loads complete in issue order, so everything but the N issued last has
// landed.  Only for loops whose VMEM instructions are all buffer-to-LDS
// loads this code issues (any other load or store in flight would be
// counted too).
template <int N>
__device__ __forceinline__ void dma_wait_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace gk
