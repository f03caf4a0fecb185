// Raw buffer loads and stores of 16-byte vectors, shared by the realignment
// kernels.  A descriptor covers one source or destination range; a lane whose
// offset lies outside it passes an out-of-range offset, which returns zero
// (load) or is dropped (store) without a memory access.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef SPECDEC_RA_AUX_LD
#define SPECDEC_RA_AUX_LD 2      // cache policy of KV loads (2 = nt: streamed, read once)
#endif
#ifndef SPECDEC_RA_AUX_ST
#define SPECDEC_RA_AUX_ST 2      // cache policy of KV stores (2 = nt)
#endif

namespace sd {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOOB = 0x80000000u;       // above every descriptor's range
constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ i32x4 bld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SPECDEC_RA_AUX_LD);
}
__device__ __forceinline__ void bst(i32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, SPECDEC_RA_AUX_ST);
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace sd
