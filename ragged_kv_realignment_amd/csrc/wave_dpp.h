// Wave- and block-level reductions and scans for the verification kernels
// (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>
#include "device_common.h"

namespace sd {

// Wave-level reductions and scans through DPP lane moves (wave64, GFX9 DPP
// controls), which stay in the vector unit; the LDS lane permutes of generic
// shuffles cost several times as much latency in these short kernels.  fp64
// values move as two 32-bit halves; lanes with no source take 0 (the `old`
// operand).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long v = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, ROW_MASK, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Inclusive prefix sum over the wave's lanes in a fixed order: within each row
// of 16 lanes by shifts of 1, 2, 4 and 8, then row 0's total into row 1 and
// row 2's into row 3, then rows 0-1's total into rows 2 and 3.
__device__ __forceinline__ double wave_scan_f64(double x) {
  x += dpp_f64<0x111, 0xF>(x);  // row_shr:1
  x += dpp_f64<0x112, 0xF>(x);  // row_shr:2
  x += dpp_f64<0x114, 0xF>(x);  // row_shr:4
  x += dpp_f64<0x118, 0xF>(x);  // row_shr:8
  x += dpp_f64<0x142, 0xA>(x);  // row_bcast:15
  x += dpp_f64<0x143, 0xC>(x);  // row_bcast:31
  return x;
}

__device__ __forceinline__ double lane_f64(double x, int lane) {
  const long long v = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)v, lane), hi = __builtin_amdgcn_readlane((int)(v >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// The wave's sum (the last lane of the scan), the same in every lane.
__device__ __forceinline__ double wave_total_f64(double x) { return lane_f64(wave_scan_f64(x), kWave - 1); }

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_f32(float x) {
  const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK, 0xF, false);
  return fmaxf(x, __int_as_float(y));
}

// The wave's maximum, the same in every lane: quad swaps, half-row and row
// mirrors, then the row broadcasts carry each row's maximum into the last row.
__device__ __forceinline__ float wave_max_f32(float v) {
  v = dpp_max_f32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_f32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_f32<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_f32<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_f32<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_max_f32<0x143, 0xC>(v);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Block sum in a fixed order: wave sums, then the wave totals in wave order.
template <int NT>
__device__ __forceinline__ double block_sum_d(double x, double *scratch) {
  x = wave_total_f64(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = x;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int k = 1; k < NT / kWave; ++k) r += scratch[k];
  return r;
}

template <int NT>
__device__ __forceinline__ float block_max_f32(float x, float *scratch) {
  x = wave_max_f32(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[threadIdx.x / kWave] = x;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int k = 1; k < NT / kWave; ++k) r = fmaxf(r, scratch[k]);
  return r;
}

// The lowest (block_first) or highest (block_last) thread of the workgroup
// whose predicate holds, by one ballot per wave: INT_MAX or -1 if none.
template <int NT>
__device__ __forceinline__ int block_first(bool pred, int *scratch) {
  const unsigned long long m = __ballot(pred);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0)
    scratch[threadIdx.x / kWave] = m ? (int)(threadIdx.x & ~(kWave - 1)) + __builtin_ctzll(m) : INT_MAX;
  __syncthreads();
  int r = INT_MAX;
#pragma unroll
  for (int k = 0; k < NT / kWave; ++k) r = min(r, scratch[k]);
  return r;
}

template <int NT>
__device__ __forceinline__ int block_last(bool pred, int *scratch) {
  const unsigned long long m = __ballot(pred);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0)
    scratch[threadIdx.x / kWave] = m ? (int)(threadIdx.x & ~(kWave - 1)) + 63 - __builtin_clzll(m) : -1;
  __syncthreads();
  int r = -1;
#pragma unroll
  for (int k = 0; k < NT / kWave; ++k) r = max(r, scratch[k]);
  return r;
}

}  // namespace sd
