// Kernel launchers called by the C ABI layer after host-side validation.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "realign_params.h"

namespace sd {

struct GreedyParams {
  const void *logits;
  int dtype;
  int64_t row_stride;
  int B, D, V;
  const int32_t *draft;
  int32_t *accept_len, *next_token, *target_tok;
  // workspace, one kAtomicLine-byte line per word: keys[r * kKeyStride] for
  // r < B*(D+1), counters[b * kCountStride] for b < B
  unsigned long long *keys;
  unsigned int *counters;
  int32_t *status;
  bool vec;                   // 16-byte aligned rows: vector loads
};

// Words that many workgroups update with device-scope atomics each get a
// 128-byte line of their own: atomics that share a line are serialized by the
// memory system, so packed words queue for microseconds where a lone word's
// round trip takes a few hundred nanoseconds.
constexpr int kAtomicLine = 128;
constexpr int kKeyStride = kAtomicLine / 8;
constexpr int kCountStride = kAtomicLine / 4;

struct SampleParams {
  const float *p, *q;
  int B, D, V;
  int R, S;                   // ids per run, splits (workgroups) per batch row
  const int32_t *draft;
  const float *u_accept, *u_draw;
  int32_t *accept_len, *next_token, *status;
  // workspace: one block of kSampleRowBytes per batch row, at a place that
  // depends on the row alone: a counter line (zero between calls), then the
  // (residual, p) mass of each of the row's S splits (kSampleSplits slots),
  // then of each of its S * kSampleThreads runs
  char *ws;
};

constexpr int kSampleThreads = 256;  // threads per sampled-verification workgroup (one run each)
constexpr int kSampleSplits = 16;    // workgroups per batch row at most (runs grow with V beyond 32768)
constexpr size_t kSampleRowBytes = kAtomicLine + (size_t)kSampleSplits * 16 + (size_t)kSampleSplits * kSampleThreads * 16;
void sample_shape(int V, int &R, int &S);

struct SampleLogitsParams {
  const void *target, *draftl;  // logits [B][D+1][V] and [B][D][V] of `dtype`
  int dtype, B, D, V;
  int S;                        // splits of kSlChunk logits per stop row (mass and draw)
  int Ss;                       // splits of kSlStatChunk logits per row (statistics)
  double inv_t;                 // 1 / temperature
  float top_p;                  // nucleus mass, in (0, 1]
  bool nucleus;                 // top_p < 1: cut every row to its nucleus
  bool vec;                     // rows 16-byte aligned: vector loads
  const int32_t *draft;
  const float *u_accept, *u_draw;
  int32_t *accept_len, *next_token, *status;
  double *stats;                // workspace [B][2D+1][Ss] x (max, exp-sum)
  float *gath;                  // workspace [B][D] x (target logit, draft logit) at the draft token
  double *part;                 // workspace [B][S] x (residual mass, target mass) of the stop row
  double *thr;                  // workspace [B][S][kSlThreads] x the same per thread run
  double *rowinfo;              // workspace [B] x 8: (M, 1/Z) of the stop row's target and draft rows,
                                // their nucleus thresholds, the draw's uniform, the stop position
  double *nuc;                  // workspace [B][2D+1] x 4: (M, 1/Z, threshold) of every nucleus
  float *cutoff;                // optional out [B][2D+1]: every row's threshold (-inf: no nucleus)
};

// Sampled verification from logits.  The statistics kernel reads each row in
// splits of kSlStatChunk logits (kSlStatThreads threads of kSlStatPer logits);
// the mass and draw kernels cut the stop row into splits of kSlChunk logits, a
// run of kSlChunk / kSlThreads consecutive ids per thread.  Compile-time knobs
// (measured defaults).
#ifndef SPECDEC_SL_STAT_THREADS
#define SPECDEC_SL_STAT_THREADS 256
#endif
#ifndef SPECDEC_SL_STAT_PER
#define SPECDEC_SL_STAT_PER 16
#endif
#ifndef SPECDEC_SL_THREADS
#define SPECDEC_SL_THREADS 512
#endif
#ifndef SPECDEC_SL_CHUNK
#define SPECDEC_SL_CHUNK 4096
#endif
constexpr int kSlStatThreads = SPECDEC_SL_STAT_THREADS;
constexpr int kSlStatPer = SPECDEC_SL_STAT_PER;
constexpr int kSlStatChunk = kSlStatThreads * kSlStatPer;
constexpr int kSlChunk = SPECDEC_SL_CHUNK;
constexpr int kSlThreads = SPECDEC_SL_THREADS;



constexpr int kPagedAppend = 0, kPagedGather = 1, kPagedAdmit = 2, kPagedRetire = 3;
constexpr int kPagedMaxGrid = 4096;   // workgroups of one append or admit launch at most
// Arrival counting of append / admit: workgroups in groups of kArriveGroup
// consecutive ids, one counter line per group plus the root line (group
// sizes 8 to 64 measured alike on MI355X).
constexpr int kArriveGroup = 32;
constexpr int kSyncStride = kAtomicLine / 4;  // int32 words between two counters
constexpr int kPagedSyncWords = (1 + kPagedMaxGrid / kArriveGroup) * kSyncStride;

struct PagedParams {
  int op;                      // kPaged*
  void *pages;                 // [L][2][n_pages][H][page][units * 16 bytes]
  int32_t *bt;                 // [rows][max_blocks] page ids, -1 = none
  int32_t *free_pages;         // [n_pages] free-page stack
  int32_t *n_free;             // [1] entries of the stack in use
  int32_t *tokens;             // [rows][max_blocks * page]
  int32_t *len;                // [rows]
  int32_t *sync;               // [kPagedSyncWords] arrival counters of append / admit (one per
                               // kSyncStride words), zero between calls
  int layers, heads, units, n_pages, page, max_blocks, rows;
  const int32_t *rowmap;       // [B] pool row of each batch entry, nullable = identity
  int B, D;
  const void *kv_new;          // append: [L][2][B][H][D+1][units * 16 bytes]
  const int32_t *draft, *accept_len, *next_token;
  int32_t pad_token;
  // the rectangle side: the view an append writes, a gather's output, an admit's input
  void *rect_kv;               // [L][2][B][H][rect_cap][units * 16 bytes]
  int32_t *rect_tok, *rect_pos, *rect_len, *rect_width;
  int8_t *rect_mask;
  int rect_cap;
  const int32_t *in_len, *in_width;  // admit: content lengths [B] and the rectangle's width [1]
  int32_t *width_out;          // append: S'
  int32_t *status;
  int kv_wgs;                  // workgroups that copy KV (set by the launcher)
};

struct GroupParams {
  const int32_t *len;
  const int32_t *ids;          // nullable: entry i is pool row ids[i] (len read there, order lists ids)
  int N, group;
  int32_t *order, *uniform, *width, *n_uniform;
};

constexpr int kMaxPoolSlots = 4096;  // pool rows a grouping or a lifecycle call handles

struct PoolParams {
  // the pool (left-aligned rows)
  void *kv;                    // [L][2][slots][H][cap][units * 16 bytes]
  int32_t *tokens, *len;       // [slots][cap], [slots]
  int layers, heads, units, slots, cap;
  // scheduling state
  int32_t *active, *n_active, *free_slots, *n_free, *q_head;
  // finish
  const int32_t *rows, *accept_len;
  int B, D;
  int32_t eos_id, max_len;
  int32_t *retired, *n_retired;
  // admit: the prompt queue [L][2][Q][H][pcap][units * 16 bytes], tokens [Q][pcap], lengths [Q]
  const void *pkv;
  const int32_t *ptok, *plen;
  int Q, pcap;
  int32_t *admitted, *n_admitted;
  int32_t *status;
};

hipError_t launch_verify_greedy(const GreedyParams &p, hipStream_t s);
hipError_t launch_verify_sample(const SampleParams &p, hipStream_t s);
hipError_t launch_verify_sample_logits(const SampleLogitsParams &p, hipStream_t s);
hipError_t launch_group_by_len(const GroupParams &p, hipStream_t s);
hipError_t launch_paged(const PagedParams &p, hipStream_t s);
hipError_t launch_pool_finish(const PoolParams &p, hipStream_t s);
hipError_t launch_pool_admit(const PoolParams &p, hipStream_t s);
hipError_t launch_zero(void *ptr, size_t bytes, hipStream_t s);
hipError_t static_scratch(void **out, hipStream_t s);

}  // namespace sd
