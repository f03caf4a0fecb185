// Parameters and launchers of the contiguous-cache realignment kernels
// (EQSPEC out of place and in place, the pool gather and append), kept apart
// from the other kernels' parameters so that those can change without
// touching the realignment kernels' sources.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

constexpr int kMaxRealignRows = 1024;  // B limit of every realignment mode

struct RealignParams {
  int mode;
  // source / destination KV in 16-byte units
  const void *kv_in;
  void *kv_out;
  const void *kv_new;
  int layers, heads, units;   // units = 16-byte units per position (head_dim * esize / 16)
  int rows_in, cap_in, rows_out, cap_out;
  const int32_t *tok_in, *len_in, *width_in;
  int32_t *tok_out, *pos_out, *len_out, *width_out;
  int8_t *mask_out;
  const int32_t *rows;        // GATHER / APPEND row map, nullable
  int B, group, D;
  const int32_t *skip_group;
  const int32_t *draft, *accept_len, *next_token;
  int32_t pad_token;
  int32_t *status;
};

int device_cus();
hipError_t launch_realign(const RealignParams &p, hipStream_t s);
hipError_t launch_realign_inplace(const RealignParams &p, hipStream_t s);

}  // namespace sd
