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
// (NT threads) takes part; acc, nxt and s_key (B * (D+1) keys) are LDS.
// Returns (uniformly) nonzero when a draft id lies outside [0, V).
template <int NT>
__device__ __forceinline__ int verify_finish(const unsigned long long *keys, int splits, int B, int D,
                                             const int32_t *draft, int V, unsigned long long *s_key, int *acc,
                                             int *nxt, int *s_red) {
  const int D1 = D + 1, R = B * D1;
  for (int r = threadIdx.x; r < R; r += NT) s_key[r] = 0ull;
  __syncthreads();
  for (int x = threadIdx.x; x < R * splits; x += NT) atomicMax(&s_key[x / splits], keys[x]);
  __syncthreads();
  int bad = 0;
  for (int b = threadIdx.x; b < B; b += NT) {
    int a = D;
    for (int i = 0; i < D; ++i) {
      const int d = draft[(size_t)b * D + i];
      if (d < 0 || d >= V) bad = 1;
      if (a == D && d != key_id(s_key[b * D1 + i])) a = i;
    }
    acc[b] = a;
    nxt[b] = key_id(s_key[b * D1 + a]);
  }
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
