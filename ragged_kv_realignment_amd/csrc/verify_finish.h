// Greedy verification's finish inside a consumer kernel ("Inference
// Engineering Part 5/8", sections "Draft Possible Tokens, Then Verify Them
// Together" and "One Verification Pass Can Commit Several Tokens": the choice
// at every position is the highest-scoring token; drafts are kept up to the
// first that differs; that position's choice replaces it, or is the bonus after
// a fully accepted draft).  The split-vocabulary pass leaves one 64-bit key per
// (row, split) workgroup; the kernel that consumes the accepted lengths reduces
// them itself, so no device-wide completion is needed between the two.
#pragma once
#include "device_common.h"
#include "specdec.h"

namespace sd {

constexpr int kMaxFinishRows = 2048;  // B * (D + 1) of a call whose consumer finishes verification

// Row r's choice is the id of the largest of keys[r * splits + s]; batch row b
// keeps its drafts up to the first one that differs from its row's choice
// (acc[b]), and nxt[b] is the choice there.  Every thread of the workgroup
// (NT threads) takes part; acc, nxt and s_key (B * (D+1) keys) are LDS.  All
// drafts (one (b, i) pair per thread and slot) and a batch of kFinishLoads keys
// per thread are loaded before any is used, so the whole finish costs about one
// round trip to memory.  Returns (uniformly) nonzero when a draft id lies
// outside [0, V).
constexpr int kFinishLoads = 8;
template <int NT>
__device__ __forceinline__ int verify_finish(const unsigned long long *keys, int splits, int B, int D,
                                             const int32_t *draft, int V, unsigned long long *s_key, int *acc,
                                             int *nxt, int *s_red) {
  constexpr int KD = (kMaxFinishRows + NT - 1) / NT;  // B * D < kMaxFinishRows
  const int D1 = D + 1, R = B * D1, P = B * D, total = R * splits;
  int dv[KD];
#pragma unroll
  for (int k = 0; k < KD; ++k) {
    const int j = k * NT + (int)threadIdx.x;
    dv[k] = j < P ? draft[j] : 0;
  }
  for (int r = threadIdx.x; r < R; r += NT) s_key[r] = 0ull;
  for (int b = threadIdx.x; b < B; b += NT) acc[b] = D;
  __syncthreads();
  for (int x0 = 0; x0 < total; x0 += kFinishLoads * NT) {
    unsigned long long v[kFinishLoads];
#pragma unroll
    for (int k = 0; k < kFinishLoads; ++k) {
      const int x = x0 + k * NT + (int)threadIdx.x;
      v[k] = x < total ? keys[x] : 0ull;
    }
#pragma unroll
    for (int k = 0; k < kFinishLoads; ++k) {
      const int x = x0 + k * NT + (int)threadIdx.x;
      if (x < total) atomicMax(&s_key[x / splits], v[k]);
    }
  }
  __syncthreads();
  int bad = 0;
#pragma unroll
  for (int k = 0; k < KD; ++k) {
    const int j = k * NT + (int)threadIdx.x;
    if (j < P) {
      const int b = j / D, i = j - b * D, d = dv[k];
      if (d < 0 || d >= V) bad = 1;
      if (d != key_id(s_key[b * D1 + i])) atomicMin(&acc[b], i);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += NT) nxt[b] = key_id(s_key[b * D1 + acc[b]]);
  return block_or_int<NT>(bad, s_red);
}

// The verification outputs of a finished call, written by one workgroup.
template <int NT>
__device__ __forceinline__ void verify_outputs(int B, int D, const unsigned long long *s_key, const int *acc,
                                               const int *nxt, int draft_bad, int32_t *accept_len,
                                               int32_t *next_token, int32_t *target_tok, int32_t *status) {
  for (int b = threadIdx.x; b < B; b += NT) {
    accept_len[b] = acc[b];
    next_token[b] = nxt[b];
  }
  if (target_tok)
    for (int r = threadIdx.x; r < B * (D + 1); r += NT) target_tok[r] = key_id(s_key[r]);
  if (draft_bad && threadIdx.x == 0) set_status(status, SPECDEC_S_DRAFT_RANGE);
}

}  // namespace sd
