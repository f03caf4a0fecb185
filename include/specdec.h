/* specdec.h - C ABI of the verify-and-resynchronize step of batch speculative
 * decoding on AMD Instinct MI355X (gfx950).
 *
 * One round of batched speculative decoding, as the pages define it:
 *   1. verification: the target model has scored D+1 positions of every row in
 *      one pass; each row keeps its drafts up to the first rejection and adds a
 *      replacement token, or a bonus token when all D drafts are accepted, so it
 *      commits between 1 and D+1 tokens ("Inference Engineering Part 5/8: When
 *      Speculative Decoding Backfires", sections "Draft Possible Tokens, Then
 *      Verify Them Together" and "Exactness Means Different Things For Greedy
 *      And Sampled Output");
 *   2. resynchronisation: rows that committed different counts no longer line
 *      up; EQSPEC unpads every row, appends its committed tokens and repads all
 *      rows on the left to the longest, recomputing position ids and shifting the
 *      KV cache, so that rectangular alignment and position-id contiguity hold
 *      again ("Batch Speculative Decoding Done Right", sections 2.1 and 2.2);
 *   3. EXSPEC scheduling: a pool of sequences is grouped by equal length so
 *      same-length batches need no realignment and only mixed batches are
 *      realigned (same page, section 2.3).
 *
 * Conventions for every entry point:
 *  - Pointers documented as "device" are device memory of the current HIP
 *    device; structs and scalars are host memory read during the call only.
 *  - The library allocates nothing, frees nothing and keeps no state between
 *    calls; all work is enqueued on `stream` (a hipStream_t passed as void*,
 *    NULL = the null stream).  Outputs are valid once the stream is
 *    synchronised.
 *  - Host-detected errors (the SPECDEC_E_* codes) are returned synchronously and
 *    nothing is enqueued.
 *  - Conditions only the device can see set bits of the optional device word
 *    `status` (SPECDEC_S_*, OR-ed in, never cleared by the library).  A call
 *    that sets CAPACITY or LEN_RANGE writes none of its outputs.
 *  - Results are deterministic: identical inputs give identical bytes.
 *  - Calls on different streams must not share output buffers or workspaces.
 *  - An empty batch (B = 0, or a rectangle of 0 rows) is a no-op after the
 *    checks of the call's persistent structures: nothing is written.  A buffer
 *    holding no bytes may be passed as NULL (a zero-size tensor has no
 *    address).
 */
#ifndef SPECDEC_H
#define SPECDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of logits and KV entries */
#define SPECDEC_F32 0
#define SPECDEC_F16 1
#define SPECDEC_BF16 2

/* host return codes */
#define SPECDEC_OK 0
#define SPECDEC_E_ARG (-1)       /* NULL pointer, size out of range, inconsistent shapes */
#define SPECDEC_E_DTYPE (-2)     /* element type not one of SPECDEC_F32/F16/BF16 */
#define SPECDEC_E_WORKSPACE (-3) /* workspace NULL or smaller than specdec_workspace_bytes() */
#define SPECDEC_E_ALIAS (-4)     /* an output overlaps an input it must not overlap */
#define SPECDEC_E_ALIGN (-5)     /* a KV position (head_dim * element size) is not a multiple of 16 bytes,
                                    or a KV/kv_new base pointer is not 16-byte aligned */
#define SPECDEC_E_LAUNCH (-6)    /* the HIP runtime refused a launch */
#define SPECDEC_E_SCRATCH (-7)   /* the call needs more workspace than the library's static scratch holds */

/* device status bits */
#define SPECDEC_S_DRAFT_RANGE 1  /* a draft id outside [0, V) (it never matches; results still written) */
#define SPECDEC_S_CAPACITY 2     /* a row would grow past its buffer's cap: nothing written */
#define SPECDEC_S_LEN_RANGE 4    /* a length outside [0, width] / [0, cap], an accepted length outside
                                    [0, D] or a row id outside the pool: nothing written */
#define SPECDEC_S_PROB 8         /* sampled verification met a position whose probabilities are all 0 */
#define SPECDEC_S_ROWS_DUP 16    /* append: the same pool row listed twice (result undefined) */

/* Library version string, e.g. "specdec 0.1 gfx950". */
const char *specdec_version(void);

/* ------------------------------------------------------------------ verify */

/* Bytes of the workspace specdec_verify_greedy needs for B rows and D drafts:
 * one 128-byte line for each of its B*(D+1) keys and B batch-row counters (a
 * base aligned to 128 bytes keeps every one of them on a line of its own;
 * 8-byte alignment is the requirement).  Returns 0 for sizes the verification
 * rejects: B or D negative, D > 255, or B*(D+1) > 2^24. */
size_t specdec_workspace_bytes(int B, int D);

/* Clears a workspace (device memory, ws_bytes >= specdec_workspace_bytes) once,
 * before its first use.  specdec_verify_greedy leaves it cleared again when it
 * completes, so the same workspace serves any number of later calls on one
 * stream. */
int specdec_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Greedy verification ("Inference Engineering Part 5/8", sections "Draft
 * Possible Tokens, Then Verify Them Together", "One Verification Pass Can
 * Commit Several Tokens" and, for greedy exactness, "Exactness Means Different
 * Things For Greedy And Sampled Output").
 *
 *  logits      device, element type `dtype`, rows (b, i) for b < B, i <= D at
 *              logits + (b*(D+1) + i) * row_stride elements; V entries per row.
 *              Row i < D scores draft i; row D gives the bonus token.
 *  row_stride  elements between consecutive rows, >= V.
 *  draft       device int32 [B][D].
 *  accept_len  device int32 [B] out: number of leading drafts equal to the
 *              target's choice, in [0, D].
 *  next_token  device int32 [B] out: the target's choice at position
 *              accept_len (the replacement, or the bonus when accept_len = D).
 *  target_tok  device int32 [B][D+1] out, nullable: the target's choice at
 *              every position.
 *  ws          device workspace, cleared once by specdec_workspace_init.
 *  status      device int32, nullable (SPECDEC_S_DRAFT_RANGE).
 * The target's choice is the id of the largest logit, the lowest such id on
 * ties; -0.0 and +0.0 are equal; NaN logits are outside the contract.
 * B = 0 is a no-op.  Errors: E_ARG (B < 0, D < 0, D > 255, V < 1, row_stride < V,
 * NULL logits/draft/outputs), E_DTYPE, E_WORKSPACE, E_LAUNCH. */
int specdec_verify_greedy(const void *logits, int dtype, int64_t row_stride, int B, int D, int V,
                          const int32_t *draft, int32_t *accept_len, int32_t *next_token,
                          int32_t *target_tok, void *ws, size_t ws_bytes, int32_t *status, void *stream);

/* Bytes of the device array that backs specdec_verify_greedy_noalloc: 4 MiB,
 * held by every GPU the library runs on until the process ends. */
#define SPECDEC_STATIC_SCRATCH_BYTES (4u << 20)

/* Greedy verification for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops and harnesses that forbid allocation):
 * specdec_verify_greedy with its workspace taken from a device array inside
 * the library instead of from the caller.  Arguments, results, status bits and
 * errors are those of specdec_verify_greedy, with no ws / ws_bytes.
 *  - The call allocates and frees nothing.  The first call on a device looks
 *    up that device's copy of the array and clears it with a fill kernel on
 *    `stream`; every call leaves it cleared again.
 *  - Limit: specdec_workspace_bytes(B, D) <= SPECDEC_STATIC_SCRATCH_BYTES, i.e.
 *    B * (D + 2) <= 32768 lines of 128 bytes; larger batches return
 *    SPECDEC_E_SCRATCH before anything is enqueued.
 *  - Every call on one device shares that device's array: calls that may run
 *    at the same time on one device (different streams, or a captured graph
 *    replayed beside an eager call) race and must be serialised by the caller.
 * Errors: those of specdec_verify_greedy except E_WORKSPACE, plus E_SCRATCH;
 * E_LAUNCH also when the array's address cannot be looked up. */
int specdec_verify_greedy_noalloc(const void *logits, int dtype, int64_t row_stride, int B, int D, int V,
                                  const int32_t *draft, int32_t *accept_len, int32_t *next_token,
                                  int32_t *target_tok, int32_t *status, void *stream);

/* Bytes of the workspace specdec_verify_sample needs for B rows: B blocks of
 * 65,920 bytes, one per batch row at a place that depends on the row alone (a
 * 128-byte counter line, 16 bytes for each of the row's at most 16 splits, then
 * 16 bytes for each of its at most 16 x 256 runs of ids).  A workspace sized for B rows therefore serves any later call
 * with at most B rows, whatever its D and V.  Returns 0 for sizes the call
 * rejects (B < 0, D < 0, V < 1, B or V > 2^30). */
size_t specdec_verify_sample_workspace_bytes(int B, int D, int V);

/* Sampled verification (speculative sampling; "Inference Engineering Part
 * 5/8", section "Exactness Means Different Things For Greedy And Sampled
 * Output": accept with probability min(1, p(x)/q(x)), replace from
 * normalize(max(0, p - q)), bonus from the target distribution after the full
 * draft).
 *
 *  p           device fp32 [B][D+1][V]: target probabilities at each position.
 *  q           device fp32 [B][D][V]: draft probabilities of each draft position.
 *  draft       device int32 [B][D].
 *  u_accept    device fp32 [B][D], uniforms in [0, 1): draft i is accepted iff
 *              u_accept[i] * q(x) <= p(x), evaluated exactly (fp64 product of
 *              fp32 values); q(x) = 0 accepts iff p(x) > 0.  A draft id outside
 *              [0, V) is rejected and sets SPECDEC_S_DRAFT_RANGE.
 *  u_draw      device fp32 [B][D+1]: u_draw[a] draws the token at stop position a
 *              by inverse CDF: w = max(0, p - q) at a < D, or p at a = D, summed
 *              in fp64; the token is the smallest id whose cumulative mass
 *              exceeds u * sum(w).  A zero sum falls back to p; an all-zero row
 *              gives id 0 and SPECDEC_S_PROB.
 *  accept_len, next_token  device int32 [B] out, as for greedy verification.
 *  ws          device workspace of at least
 *              specdec_verify_sample_workspace_bytes(B, D, V) bytes, 16-byte
 *              aligned, cleared once by specdec_workspace_init; every call
 *              leaves its counters cleared again.
 * Each batch row is spread over up to 16 workgroups; the last to finish draws.
 * B = 0 is a no-op.  Errors: E_ARG (also D > 255), E_WORKSPACE, E_LAUNCH. */
int specdec_verify_sample(const float *p, const float *q, int B, int D, int V, const int32_t *draft,
                          const float *u_accept, const float *u_draw, int32_t *accept_len,
                          int32_t *next_token, void *ws, size_t ws_bytes, int32_t *status, void *stream);

/* Bytes of the workspace specdec_verify_sample_logits needs for B rows, D
 * drafts and V logits per row. */
size_t specdec_sample_workspace_bytes(int B, int D, int V);

/* Sampled verification from logits: the rule of specdec_verify_sample with p
 * and q formed from logits by the sampling settings ("Inference Engineering
 * Part 5/8", opening section: the decoding rule may sample using temperature
 * and top-p; section "Exactness Means Different Things For Greedy And Sampled
 * Output": the draft and the target use the same settings).
 *
 *  target        device [B][D+1][V] target logits of element type `dtype`.
 *  draft_logits  device [B][D][V] draft-model logits of the same type.
 *  temperature   > 0 and finite: e(v) = exp((l(v) - M) / T) with M the row
 *                maximum, with about 1e-7 relative error (the exponent formed
 *                in fp64 from an exact difference, 2^f of its fraction by the
 *                hardware's fp32 exp2); sums and comparisons in fp64.
 *  top_p         in (0, 1].  Below 1 every row (target and draft alike) is cut
 *                to its nucleus: the ids whose logit is at least t, where t is
 *                the largest logit value such that the ids at or above it hold
 *                at least top_p of the row's mass sum(e); every id tied at t is
 *                kept.  The masses deciding t carry the relative error of e
 *                (about 1e-7) and are summed exactly as integer multiples of
 *                2^-41 (of the maximum's mass), so t differs from an fp64
 *                evaluation only where the mass above a value is within about
 *                1e-7 relative (plus V * 2^-42) of top_p * sum(e).  At 1 every
 *                id is kept.
 *                p(v) = e(v) / Z over the kept ids (Z in fp64), 0 elsewhere.
 *  draft, u_accept, u_draw, accept_len, next_token, status
 *                as for specdec_verify_sample; the acceptance test and the
 *                draw compare fp64 values formed on the device.
 *  cutoff        nullable device float [B][2D+1] out: the threshold t applied
 *                to each row, the D+1 target rows of a batch row before its D
 *                draft rows (-inf when every id is kept).
 *  ws            device workspace of at least specdec_sample_workspace_bytes
 *                (B, D, V) bytes, 16-byte aligned; scratch only, nothing is
 *                kept between calls.  Calls that share a workspace must not
 *                overlap.
 * Logits are finite or -inf with at least one finite value per row; NaN is
 * outside the contract.  B = 0 is a no-op.  Errors: E_ARG (B outside
 * [0, 65535], D outside [0, 255], V outside [1, 2^22], temperature or top_p out
 * of range, NULL pointers), E_DTYPE, E_WORKSPACE, E_ALIGN, E_LAUNCH. */
int specdec_verify_sample_logits(const void *target, const void *draft_logits, int dtype, int B, int D, int V,
                                 float temperature, float top_p, const int32_t *draft, const float *u_accept,
                                 const float *u_draw, int32_t *accept_len, int32_t *next_token, float *cutoff,
                                 void *ws, size_t ws_bytes, int32_t *status, void *stream);

/* --------------------------------------------------------------- realign */

/* A set of sequences with a contiguous KV cache.
 *  kv        device [layers][2 (K, V)][rows][heads][cap][head_dim] of `dtype`;
 *            each (layer, K|V, row, head) sequence of cap positions is
 *            contiguous, one position = head_dim elements.
 *  tokens    device int32 [rows][cap] token ids.
 *  pos       device int32 [rows][cap] position ids (nullable for a pool).
 *  mask      device int8 [rows][cap] attention mask, 1 = content (nullable for
 *            a pool).
 *  len       device int32 [rows] content length of each row.
 *  width     device int32: [1] the rectangle width of a left-padded batch, or
 *            [groups] one width per rectangle of a GATHER output (NULL for a
 *            pool).
 * A left-padded rectangle of width S holds row b's content at positions
 * [S - len[b], S); a pool holds it at [0, len[b]). */
typedef struct {
  void *kv;
  int32_t *tokens;
  int32_t *pos;
  int8_t *mask;
  int32_t *len;
  int32_t *width;
  int32_t rows, cap, layers, heads, head_dim;
  int32_t dtype;
} specdec_seqbuf_t;

#define SPECDEC_EQSPEC 0         /* rectangle -> rectangle: unpad, append, repad (out of place) */
#define SPECDEC_GATHER 1         /* pool rows -> one left-padded rectangle per group (no append) */
#define SPECDEC_APPEND_INPLACE 2 /* pool rows: append committed entries at each row's length */
#define SPECDEC_EQSPEC_INPLACE 3 /* rectangle -> the same rectangle: unpad, append, repad in place */
#define SPECDEC_EQSPEC_INPLACE_ZERO_PAD 4 /* as SPECDEC_EQSPEC_INPLACE, for an input whose pad may hold any bytes */

/* Realignment ("Batch Speculative Decoding Done Right", sections 2.1-2.3;
 * committed and discarded speculative KV: "Inference Engineering Part 5/8",
 * section "Acceptance changes across the workload").
 *
 * Row b commits n_b = accept_len[b] + 1 tokens: draft[b][0 .. accept_len-1]
 * then next_token[b], with the first n_b of its D+1 speculative KV entries
 * kv_new [layers][2][B][heads][D+1][head_dim] (device, same type as the cache).
 *
 * SPECDEC_EQSPEC: `in` is a left-padded rectangle of B = in->rows rows and
 *   width in->width[0]; `out` receives the rectangle of width
 *   S' = max_b(len[b] + n_b): row b's old content, then its committed entries,
 *   left-padded with zero KV bytes, pad_token, position id 0 and mask 0.
 *   Position ids are 0..len-1 over the content.  out->len and out->width[0] are
 *   written; positions [S', cap) of `out` are not touched.  in and out must
 *   not overlap (E_ALIAS).  rows / group / skip_group are unused (NULL / 0).
 * SPECDEC_GATHER: `in` is a pool; rows[j] (NULL = j) names the pool row of
 *   batch entry j < B; entries form groups of `group` consecutive entries.
 *   Every group whose skip_group[g] is 0 (skip_group NULL = none skipped) is
 *   written to `out` (a rectangle buffer with out->rows >= B) as a left-padded
 *   rectangle of width W_g = its longest row: out row j gets pool row rows[j]'s
 *   content and tokens, with mask, position ids, out->len[j] and
 *   out->width[g].  Skipped groups are not touched.  D, kv_new, draft,
 *   accept_len, next_token are unused.
 * SPECDEC_APPEND_INPLACE: `in` and `out` describe the same pool (same kv,
 *   tokens, len); batch entry b < B (pool row rows[b], NULL = b) appends its
 *   committed entries and tokens at its length, and its length grows by n_b.
 *   Rows must be distinct (else SPECDEC_S_ROWS_DUP and an undefined result).
 * SPECDEC_EQSPEC_INPLACE: the EQSPEC result on positions [0, S') of the same
 *   rectangle (`in` and `out` describe identical buffers).  Each row's content
 *   moves by S' - S - n_b positions; rows whose shift is 0 only append.  The
 *   input's pad positions must hold zero KV bytes (every realignment leaves
 *   them so); positions [S', cap) keep their previous bytes.  Moves only the
 *   bytes that change: about twice each shifted row's content, its committed
 *   entries and any newly exposed pad, instead of the whole new rectangle.
 *   Device conditions as for EQSPEC; a failing call writes nothing.
 * SPECDEC_EQSPEC_INPLACE_ZERO_PAD: SPECDEC_EQSPEC_INPLACE for a rectangle whose
 *   pad positions may hold any KV bytes (a left-padded prefill writes KV at its
 *   pad positions): every row's new pad [0, S' - len - n_b) is written with zero
 *   bytes, so the result equals EQSPEC's on [0, S') whatever the input pad held.
 *   It writes P * sum_b min(pad_b, pad'_b) bytes more than SPECDEC_EQSPEC_INPLACE
 *   (P the KV bytes of one position over layers, K|V and heads); use it for the
 *   first round after such a prefill, after which the pad is zero.
 * Limits: B <= 1024; head_dim * element size a multiple of 16 bytes; KV
 * pointers 16-byte aligned (E_ALIGN).  Device conditions: S' > out cap,
 * W_g > out cap or len + n_b > cap set SPECDEC_S_CAPACITY; lengths outside
 * [0, width] (EQSPEC) or [0, cap], accepted lengths outside [0, D] or rows
 * outside the pool set SPECDEC_S_LEN_RANGE; either way nothing is written.
 * Errors: E_ARG, E_DTYPE, E_ALIAS, E_ALIGN, E_LAUNCH. */
int specdec_realign_kv(int mode, const specdec_seqbuf_t *in, const specdec_seqbuf_t *out,
                       const int32_t *rows, int B, int group, const int32_t *skip_group, int D,
                       const void *kv_new, const int32_t *draft, const int32_t *accept_len,
                       const int32_t *next_token, int32_t pad_token, int32_t *status, void *stream);

/* Equal-length grouping of a sequence pool ("Batch Speculative Decoding Done
 * Right", section 2.3: batches of same-length sequences need no realignment).
 *
 *  len        device int32 [N] content lengths, N <= 4096.
 *  group      rows per batch (>= 1).
 *  order      device int32 [N] out: pool ids in batch-major order.  Ids are
 *             ranked by (length, id); for each length in ascending order the
 *             first floor(count / group) * group ids form full same-length
 *             batches, listed first; the remaining ids follow in (length, id)
 *             order and are cut into batches of `group` (the last may be short).
 *  uniform    device int32 [ceil(N / group)] out: 1 if every length in the
 *             batch is equal (such a batch needs no realignment).
 *  width      device int32 [ceil(N / group)] out: longest length in the batch.
 *  n_uniform  device int32 [1] out: number of uniform batches.
 * Errors: E_ARG (N < 0, N > 4096, group < 1, NULL outputs), E_LAUNCH. */
int specdec_group_by_len(const int32_t *len, int N, int group, int32_t *order, int32_t *uniform,
                         int32_t *width, int32_t *n_uniform, void *stream);

/* Equal-length grouping over a list of pool rows: as specdec_group_by_len with
 * entry i the pool row ids[i] (device int32 [N]): its length is len[ids[i]]
 * (len: device int32, one entry per pool row), and `order` lists pool rows
 * (ids entries) instead of indices.  Errors as for specdec_group_by_len, and
 * E_ARG for a NULL ids. */
int specdec_group_by_len_ids(const int32_t *len, const int32_t *ids, int N, int group, int32_t *order,
                             int32_t *uniform, int32_t *width, int32_t *n_uniform, void *stream);

/* --------------------------------------------------------- pool lifecycle */

/* Scheduling state of a pool of sequences ("Batch Speculative Decoding Done
 * Right", section 2.3: EXSPEC keeps a pool of active sequences, not a fixed
 * batch).  All device int32:
 *  active      [slots]: the active sequences' pool rows in schedule order;
 *              entries [0, *n_active) are valid.
 *  n_active    [1].
 *  free_slots  [slots]: the free pool rows in ascending order; entries
 *              [0, *n_free) are valid.
 *  n_free      [1].
 *  q_head      [1]: the next prompt of the queue to admit.
 * Every pool row is active or free, never both.  The pool (specdec_seqbuf_t)
 * is left-aligned: row s holds its content at positions [0, len[s]). */
typedef struct {
  int32_t *active;
  int32_t *n_active;
  int32_t *free_slots;
  int32_t *n_free;
  int32_t *q_head;
} specdec_sched_t;

/* Finish after a round's append: rows [B] (device) is the round's batch order,
 * a permutation of the active list (B == *n_active), and accept_len [B] its
 * accepted lengths (entry j committed accept_len[j] + 1 tokens, now the last
 * ones of row rows[j]).  A sequence finishes at the first newly committed
 * position p holding eos_id, or with p + 1 >= max_len (max_len >= 1): its
 * length becomes p + 1, it leaves the active list (the others keep their
 * order) and its row joins the free rows.  retired [pool->rows] (device)
 * receives the finished rows in active-list order and *n_retired (device) their
 * count.  Device conditions (nothing written): B != *n_active, rows outside the
 * pool or not active, accepted lengths outside [0, D], a length shorter than its
 * committed tokens set SPECDEC_S_LEN_RANGE; a row twice SPECDEC_S_ROWS_DUP.
 * Limits: pool->rows <= 4096.  Errors: E_ARG, E_LAUNCH. */
int specdec_pool_finish(const specdec_seqbuf_t *pool, const specdec_sched_t *sched, const int32_t *rows,
                        const int32_t *accept_len, int B, int D, int32_t eos_id, int32_t max_len, int32_t *retired,
                        int32_t *n_retired, int32_t *status, void *stream);

/* Admit from a prompt queue: `queue` holds Q = queue->rows prompts in the
 * pool's geometry, left-aligned (prompt q's content at [0, queue->len[q]) of its
 * row, token ids in queue->tokens).  The next k = min(*n_free, Q - *q_head)
 * prompts, in queue order, go to the k lowest free rows and join the end of the
 * active list; their content and token ids are copied and their lengths set.
 * admitted [pool->rows] (device) receives the rows filled, in order, and
 * *n_admitted (device) k.  Device conditions (nothing admitted, *n_admitted =
 * 0): a prompt longer than pool->cap sets SPECDEC_S_CAPACITY; inconsistent
 * counts or lengths outside [0, queue->cap] SPECDEC_S_LEN_RANGE.
 * An empty queue (queue->rows = 0) admits nothing.
 * Limits: pool->rows <= 4096.  Errors: E_ARG, E_DTYPE, E_ALIGN, E_ALIAS,
 * E_LAUNCH. */
int specdec_pool_admit(const specdec_seqbuf_t *pool, const specdec_sched_t *sched, const specdec_seqbuf_t *queue,
                       int32_t *admitted, int32_t *n_admitted, int32_t *status, void *stream);

/* ------------------------------------------------------------- paged KV */

/* A paged KV cache: rows of sequences whose positions live in pages of a
 * shared pool, listed per row in a block table.  The arXiv abstract of "Batch
 * Speculative Decoding Done Right" ties the superlinear cost of realignment
 * to contiguous layouts; with a block table the left-padded rectangle that
 * section 2.1 requires (equal pad + content length for every row, position ids
 * 0.. over the content) is metadata, pad = S' - len, and section 2.2's
 * unpad-append-repad writes only each row's committed entries.
 *  pages        device [layers][2 (K, V)][n_pages][heads][page][head_dim] of
 *               `dtype`: row r's content position j is in page
 *               block_table[r][j / page], slot j % page.
 *  block_table  device int32 [rows][max_blocks]: page ids of each row's blocks
 *               in order; -1 past the row's ceil(len / page) blocks.
 *  free_pages   device int32 [n_pages]: a stack of free page ids; entries
 *               [0, *n_free) are free.
 *  n_free       device int32 [1].
 *  tokens       device int32 [rows][max_blocks * page]: each row's token ids
 *               from position 0.
 *  len          device int32 [rows]: content length of each row.
 *  sync         device int32 [SPECDEC_PAGED_SYNC_WORDS]: zero when the cache is
 *               created; append and admit count their workgroups in it (one
 *               counter per 128-byte line) and leave it zero.
 * Calls on one cache must not overlap (they are stream-ordered on one stream).
 * Allocation: batch entries in order take their new pages from the top of the
 * free stack, an entry's first new block getting the topmost remaining id;
 * retiring pushes a row's pages back in block order, entries in batch order.
 * Every page is free or in exactly one row's table; the calls keep it so. */
#define SPECDEC_PAGED_SYNC_WORDS 4128

typedef struct {
  void *pages;
  int32_t *block_table;
  int32_t *free_pages;
  int32_t *n_free;
  int32_t *tokens;
  int32_t *len;
  int32_t *sync;
  int32_t rows, n_pages, page, max_blocks, layers, heads, head_dim;
  int32_t dtype;
} specdec_paged_t;

/* Realignment on a paged cache.  Batch entry b (pool row rows[b], NULL = b;
 * rows distinct, else SPECDEC_S_ROWS_DUP and an undefined result) commits
 * n_b = accept_len[b] + 1 tokens, draft[b][0 .. accept_len-1] then
 * next_token[b], and the first n_b of its D+1 speculative entries kv_new
 * [layers][2][B][heads][D+1][head_dim] (device, 16-byte aligned), written at
 * positions len, len+1, ... of the row; new pages come off the free stack.
 * No other KV byte moves.  The kv_new units this reads are numbered with
 * 32-bit integers: layers * 2 * B * heads * (D+1) * head_dim * element size
 * must stay below 2^35 bytes (E_ARG).  *width (device int32, nullable) receives
 * S' = max_b(len_b + n_b).  The rectangle view (rect_tokens nullable, then
 * nothing of it is written; rect_pos and rect_mask nullable; all
 * [B][rect_cap] on the device): row b left-padded by S' - len'_b with
 * pad_token, position id 0 and mask 0, then its content with position ids
 * 0.. and mask 1, on [0, S'); the same tokens, positions and mask that
 * SPECDEC_EQSPEC writes.  Device conditions (nothing written): a row past
 * max_blocks * page positions, more new pages than free ones, or S' > rect_cap
 * set SPECDEC_S_CAPACITY; rows outside [0, rows), lengths outside
 * [0, max_blocks * page], accepted lengths outside [0, D], or a page id outside
 * [0, n_pages) where the call would write set SPECDEC_S_LEN_RANGE.
 * Limits: B <= 1024.  Errors: E_ARG, E_DTYPE, E_ALIGN, E_ALIAS, E_LAUNCH. */
int specdec_paged_append(const specdec_paged_t *kv, const int32_t *rows, int B, int D, const void *kv_new,
                         const int32_t *draft, const int32_t *accept_len, const int32_t *next_token,
                         int32_t pad_token, int32_t *width, int32_t *rect_tokens, int32_t *rect_pos,
                         int8_t *rect_mask, int rect_cap, int32_t *status, void *stream);

/* The batch's rows (rows[b], NULL = b) as the left-padded rectangle of width
 * W = their longest length: out (a specdec_seqbuf_t with out->rows == B and the
 * cache's geometry) receives KV with zero bytes on the pad, token ids, position
 * ids, mask and lengths on [0, W), and out->width[0] = W; [W, out->cap) is not
 * written.  This is the rectangle SPECDEC_EQSPEC would hold.  W > out->cap sets
 * SPECDEC_S_CAPACITY and a bad row or length SPECDEC_S_LEN_RANGE (nothing
 * written); a block-table entry outside [0, n_pages) reads as zero bytes and
 * sets SPECDEC_S_LEN_RANGE.  Errors: E_ARG, E_DTYPE, E_ALIGN, E_ALIAS,
 * E_LAUNCH. */
int specdec_paged_gather(const specdec_paged_t *kv, const int32_t *rows, int B, const specdec_seqbuf_t *out,
                         int32_t pad_token, int32_t *status, void *stream);

/* Admit: the content of a left-padded rectangle `in` (in->rows == B, width
 * in->width[0] on the device, content of entry b at [width - in->len[b],
 * width), token ids in in->tokens) becomes pool rows rows[b] (NULL = b), which
 * must be empty (length 0).  Pages come off the free stack.  Device conditions
 * (nothing written): too few free pages or a row past max_blocks * page set
 * SPECDEC_S_CAPACITY; a row that is not empty, lengths outside [0, width],
 * width outside [0, in->cap] or a bad row set SPECDEC_S_LEN_RANGE.
 * Errors: E_ARG, E_DTYPE, E_ALIGN, E_ALIAS, E_LAUNCH. */
int specdec_paged_admit(const specdec_paged_t *kv, const int32_t *rows, int B, const specdec_seqbuf_t *in,
                        int32_t *status, void *stream);

/* Retire: rows rows[b] (NULL = b) give their pages back to the free stack
 * (pushed in block order, entries in batch order); their block-table entries
 * become -1 and their lengths 0.  Bad rows or lengths, or more pages than the
 * stack holds, set SPECDEC_S_LEN_RANGE; duplicate rows SPECDEC_S_ROWS_DUP
 * (nothing written either way).  Errors: E_ARG, E_LAUNCH. */
int specdec_paged_retire(const specdec_paged_t *kv, const int32_t *rows, int B, int32_t *status, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECDEC_H */
