// 16-byte loads and stores through the device's coherence point, for the
// sums one workgroup leaves for the last-arriving workgroup of a completion
// (sampled verification, from probabilities or from logits).
//
// The buffer cache policy sc1 writes a store through to, and reads a load
// from, the coherence point past the non-coherent per-XCD L2.  The writer waits
// for its stores to complete (vmcnt) before it counts itself with a returning
// atomic, and the last workgroup loads only after its own count has returned;
// see the ordering notes beside each kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

constexpr int kCoherentPolicy = 16;        // buffer cache policy bit sc1
constexpr int kCoherentRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

typedef int i32x4v __attribute__((ext_vector_type(4)));

// A buffer resource over `bytes` bytes at `base` (offsets past it read 0 and
// drop stores).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, kCoherentRsrcWord3);
}

__device__ __forceinline__ void st_pair(__amdgpu_buffer_rsrc_t r, uint32_t off, double a, double b) {
  const long long la = __double_as_longlong(a), lb = __double_as_longlong(b);
  const i32x4v v = {(int)la, (int)(la >> 32), (int)lb, (int)(lb >> 32)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCoherentPolicy);
}

__device__ __forceinline__ void ld_pair(__amdgpu_buffer_rsrc_t r, uint32_t off, double &a, double &b) {
  const i32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentPolicy);
  a = __longlong_as_double(((long long)(unsigned)v[1] << 32) | (unsigned)v[0]);
  b = __longlong_as_double(((long long)(unsigned)v[3] << 32) | (unsigned)v[2]);
}

}  // namespace sd
