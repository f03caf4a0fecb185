// Device helpers shared by the library's kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

constexpr int kBlock = 256;     // threads per workgroup: 4 waves of 64
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// (value, id) order used by the argmax: larger value wins, the lower id on equal
// values.  Float comparison makes -0.0 == +0.0.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float &bv, int &bi) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
}

// Monotone 64-bit key of (value, id): larger key = larger value, then lower id.
// -0.0 is folded onto +0.0 first so the key order matches float comparison.
__device__ __forceinline__ unsigned long long argmax_key(float v, int id) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(~(uint32_t)id);
}

__device__ __forceinline__ int key_id(unsigned long long k) { return (int)(~(uint32_t)(k & 0xFFFFFFFFull)); }

__device__ __forceinline__ unsigned long long load_agent(const unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(unsigned long long *p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(unsigned int *p, unsigned int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void set_status(int32_t *status, int32_t bits) {
  if (status && bits) atomicOr(status, bits);
}

// Block-wide reductions for kBlock threads; `scratch` holds kBlock/kWave ints.
__device__ __forceinline__ int block_max_int(int v, int *scratch) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int r = scratch[0];
#pragma unroll
  for (int k = 1; k < kBlock / kWave; ++k) r = max(r, scratch[k]);
  return r;
}

__device__ __forceinline__ int block_or_int(int v, int *scratch) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v |= __shfl_xor(v, off);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int k = 0; k < kBlock / kWave; ++k) r |= scratch[k];
  return r;
}

}  // namespace sd
