/* Reference oracle for the verify-and-resynchronize step of batch speculative
 * decoding.  TEST INFRASTRUCTURE ONLY: plain, slow C (single-threaded in the
 * build the tests load) that the tests, the smoke check and the benchmark's
 * CPU-baseline leg call to decide what the GPU path must produce.  It shares
 * no code, header or table with the GPU library and never runs on the product
 * path.
 *
 * Sources (the pages this follows):
 *  [NL]  "Inference Engineering Part 5/8: When Speculative Decoding Backfires",
 *        sections "Draft Possible Tokens, Then Verify Them Together",
 *        "One Verification Pass Can Commit Several Tokens",
 *        "Exactness Means Different Things For Greedy And Sampled Output",
 *        "Acceptance changes across the workload".
 *  [BD]  "Batch Speculative Decoding Done Right" (technical summary), section 2.1
 *        (synchronization invariants), 2.2 (EQSPEC unpad-append-repad),
 *        2.3 (EXSPEC cross-batch scheduling).
 *  [AB]  arXiv 2510.22876 abstract: invariants, contiguous layouts.
 *
 * Readings where the pages leave a choice open are stated at each function.
 * Floating point: greedy compares exactly widened values; sampled acceptance
 * and residual masses are evaluated in fp64.  Parity of every function here
 * is pinned by the CPU tests (worked examples, closed forms, brute force).
 *
 * Threads: the library the tests load is built without OpenMP and runs every
 * loop in order on one thread.  The same source built with -fopenmp
 * (liboracle_omp.so) serves only to time the oracle on all host cores: there
 * greedy verification splits its batch rows and the EQSPEC realignment its
 * (layer, K|V, row, head) KV segments over threads.  Each of those units
 * writes only its own outputs, so both builds produce the same bytes (the
 * threaded realignment additionally needs kv_out apart from kv_in). */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

/* Threads the loops below may use: 1 unless built with OpenMP. */
EXPORT int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

enum { O_F32 = 0, O_F16 = 1, O_BF16 = 2 };
enum { O_OK = 0, O_E_ARG = -1, O_E_CAPACITY = -2, O_E_PRECOND = -3 };

/* ---------------------------------------------------------------- values */

static double decode_f16(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m + 1024), e - 25);
  return s ? -v : v;
}

static double decode_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double logit_at(const void *base, int dtype, int64_t idx) {
  if (dtype == O_F32) return (double)((const float *)base)[idx];
  if (dtype == O_F16) return decode_f16(((const uint16_t *)base)[idx]);
  return decode_bf16(((const uint16_t *)base)[idx]);
}

/* -------------------------------------------------- greedy verification
 * [NL] "Exactness ...": greedy decoding picks the highest-scoring token; the
 * target's choice is compared with each draft, matches are accepted and the
 * first mismatch is replaced by the target's choice.  [NL] "Draft Possible
 * Tokens ...": results are read left to right up to the first rejection; drafts
 * after it are discarded unjudged; when all D drafts are accepted the
 * distribution after the full draft gives one more (bonus) token, so a cycle
 * commits 1..D+1 tokens.
 * Readings: logit row i (0 <= i < D) verifies draft i and row D gives the
 * bonus; ties at the maximum go to the lowest id; -0 and +0 compare equal;
 * values are compared exactly (no temperature or softmax, which cannot change
 * the argmax).  NaN logits are outside the contract. */
EXPORT int oracle_verify_greedy(const void *logits, int dtype, int64_t row_stride, int B, int D, int V,
                                const int32_t *draft, int32_t *accept_len, int32_t *next_token,
                                int32_t *target_tok) {
  if (B < 0 || D < 0 || V <= 0 || row_stride < V) return O_E_ARG;
  int32_t *targets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1) * (size_t)(D + 1));
#pragma omp parallel for schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    int32_t *t = targets + (size_t)b * (D + 1);
    for (int i = 0; i <= D; ++i) {
      const int64_t row = ((int64_t)b * (D + 1) + i) * row_stride;
      int best = 0;
      double bv = logit_at(logits, dtype, row);
      for (int v = 1; v < V; ++v) {
        const double x = logit_at(logits, dtype, row + v);
        if (x > bv) { bv = x; best = v; }
      }
      t[i] = best;
      if (target_tok) target_tok[(int64_t)b * (D + 1) + i] = best;
    }
    int a = 0;
    while (a < D && draft[(int64_t)b * D + a] == t[a]) ++a;
    accept_len[b] = a;
    next_token[b] = t[a];
  }
  free(targets);
  return O_OK;
}

/* ------------------------------------------------- sampled verification
 * [NL] "Exactness ...": a draft x proposed by the draft model with probability
 * q(x) is accepted with probability min(1, p(x)/q(x)); at the first rejection
 * the replacement is drawn from normalize(max(0, p - q)); when every draft is
 * accepted the bonus comes from the target distribution after the full draft.
 * Readings: the caller supplies the uniforms; draft i is accepted iff
 * u_accept[i] <= p(x)/q(x), evaluated as u*q <= p in fp64; q(x) = 0 accepts iff
 * p(x) > 0.  The draw at stop position a uses u_draw[a]: with w the residual
 * (a < D) or p at position D (a = D), T = sum of w in fp64 in id order, the
 * token is the smallest id whose cumulative mass exceeds u*T; if rounding
 * leaves none, the last id with w > 0.  If T is 0 the draw falls back to p at
 * that position (unreachable for normalised p and q); an all-zero row yields
 * id 0 and a return of O_E_PRECOND.
 *
 * One batch row: P holds the D+1 target rows and Q the D draft rows, V fp64
 * probabilities each; w is V doubles of scratch.  Returns 1 for an all-zero row. */
static int sample_row(const double *P, const double *Q, int D, int V, const int32_t *draft,
                      const float *u_accept, const float *u_draw, double *w, int32_t *a_out, int32_t *j_out,
                      double *mass_out) {
  int a = D;
  for (int i = 0; i < D; ++i) {
    const int32_t x = draft[i];
    int ok = 0;
    if (x >= 0 && x < V) {
      const double px = P[(int64_t)i * V + x];
      const double qx = Q[(int64_t)i * V + x];
      const double u = u_accept[i];
      ok = (qx > 0.0) ? (u * qx <= px) : (px > 0.0);
    }
    if (!ok) { a = i; break; }
  }
  const double *pa = P + (int64_t)a * V;
  const double *qa = (a < D) ? Q + (int64_t)a * V : NULL;
  double T = 0.0;
  for (int v = 0; v < V; ++v) {
    const double d = qa ? pa[v] - qa[v] : pa[v];
    w[v] = d > 0.0 ? d : 0.0;
    T += w[v];
  }
  if (!(T > 0.0)) {
    T = 0.0;
    for (int v = 0; v < V; ++v) { w[v] = pa[v] > 0.0 ? pa[v] : 0.0; T += w[v]; }
  }
  int j = -1, zero = 0;
  if (T > 0.0) {
    const double target = (double)u_draw[a] * T;
    double c = 0.0;
    for (int v = 0; v < V; ++v) {
      c += w[v];
      if (c > target) { j = v; break; }
    }
    if (j < 0)
      for (int v = V - 1; v >= 0; --v)
        if (w[v] > 0.0) { j = v; break; }
  } else {
    j = 0;
    zero = 1;
  }
  *a_out = a;
  *j_out = j;
  if (mass_out) *mass_out = T;
  return zero;
}

/* Probabilities given directly: fp32 p [B][D+1][V] and q [B][D][V], each value
 * widened exactly to fp64. */
EXPORT int oracle_verify_sample(const float *p, const float *q, int B, int D, int V, const int32_t *draft,
                                const float *u_accept, const float *u_draw, int32_t *accept_len,
                                int32_t *next_token, double *mass) {
  if (B < 0 || D < 0 || V <= 0) return O_E_ARG;
  int rc = O_OK;
  double *P = (double *)malloc(sizeof(double) * (size_t)(D + 1) * V);
  double *Q = (double *)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1) * V);
  double *w = (double *)malloc(sizeof(double) * (size_t)V);
  for (int b = 0; b < B; ++b) {
    for (int64_t k = 0; k < (int64_t)(D + 1) * V; ++k) P[k] = p[(int64_t)b * (D + 1) * V + k];
    for (int64_t k = 0; k < (int64_t)D * V; ++k) Q[k] = q[(int64_t)b * D * V + k];
    if (sample_row(P, Q, D, V, draft + (int64_t)b * D, u_accept + (int64_t)b * D, u_draw + (int64_t)b * (D + 1),
                   w, &accept_len[b], &next_token[b], mass ? &mass[b] : NULL))
      rc = O_E_PRECOND;
  }
  free(P);
  free(Q);
  free(w);
  return rc;
}

/* Sampling settings ([NL] opening section: the decoding rule may sample among
 * likely tokens using temperature and top-p; "Exactness ...": the draft and the
 * target use the same sampling settings).  Row l of V logits becomes
 * probabilities in fp64:
 *  - temperature: e(v) = exp((l(v) - M) / T) with M = max l; the maximum is
 *    subtracted so no term overflows, and the result does not depend on it;
 *  - top-p (0 < top_p < 1): the nucleus is every id whose logit is at least t,
 *    where t is the largest logit value such that the ids with logit >= t hold
 *    at least top_p of the mass sum(e); ids tied at t are all kept.  If
 *    rounding leaves the whole mass short of top_p * sum(e), every id is kept.
 *    top_p >= 1 keeps every id;
 *  - p(v) = e(v) / Z over the kept ids, 0 elsewhere; Z is summed in id order.
 * Where the mass of the ids above a candidate t lies within rounding of
 * top_p * sum(e), more than one t is correct; a caller may then give t itself
 * (`cut`), and the row is formed from that nucleus.
 * `order` is V ints of scratch. */
static const double *g_sort_key;
static int by_key_desc(const void *x, const void *y) {
  const double a = g_sort_key[*(const int *)x], b = g_sort_key[*(const int *)y];
  return a < b ? 1 : (a > b ? -1 : 0);
}

/* The nucleus threshold t for logits lv and masses e (-inf: every id kept). */
static double nucleus_cut(const double *lv, const double *e, int V, double top_p, int *order) {
  if (!(top_p < 1.0)) return -INFINITY;
  double total = 0.0;
  for (int v = 0; v < V; ++v) total += e[v];
  for (int v = 0; v < V; ++v) order[v] = v;
  g_sort_key = lv;
  qsort(order, (size_t)V, sizeof(int), by_key_desc);
  const double need = top_p * total;
  double cum = 0.0;
  int k = 0;
  while (k < V) {
    const double val = lv[order[k]];
    while (k < V && lv[order[k]] == val) cum += e[order[k++]];
    if (cum >= need) return val;
  }
  return -INFINITY;
}

/* One row: out = p; *cut_used (nullable) receives the threshold applied. */
static void softmax_row(const void *logits, int dtype, int64_t row0, int V, double T, double top_p,
                        const float *cut, double *out, double *lv, int *order, float *cut_used) {
  double M = -INFINITY;
  for (int v = 0; v < V; ++v) {
    lv[v] = logit_at(logits, dtype, row0 + v);
    if (lv[v] > M) M = lv[v];
  }
  for (int v = 0; v < V; ++v) out[v] = exp((lv[v] - M) / T);
  const double t = cut ? (double)*cut : nucleus_cut(lv, out, V, top_p, order);
  for (int v = 0; v < V; ++v)
    if (lv[v] < t) out[v] = 0.0;
  double Z = 0.0;
  for (int v = 0; v < V; ++v) Z += out[v];
  for (int v = 0; v < V; ++v) out[v] /= Z;
  if (cut_used) *cut_used = (float)t;
}

/* Logits given: target [B][D+1][V] and draft [B][D][V] of element type dtype
 * (widened exactly), turned into p and q by softmax_row with the same
 * temperature and top-p, then decided as oracle_verify_sample does.  `cut`
 * (nullable) gives every row's nucleus threshold instead, [B][2D+1] with the
 * D+1 target rows of a batch row before its D draft rows; `cut_used`
 * (nullable, same layout) receives the thresholds applied. */
EXPORT int oracle_verify_sample_logits(const void *target, const void *draftl, int dtype, int B, int D, int V,
                                       float temperature, float top_p, const float *cut, const int32_t *draft,
                                       const float *u_accept, const float *u_draw, int32_t *accept_len,
                                       int32_t *next_token, double *mass, float *cut_used) {
  if (B < 0 || D < 0 || V <= 0 || !(temperature > 0.0f) || !isfinite(temperature) || !(top_p > 0.0f) ||
      top_p > 1.0f)
    return O_E_ARG;
  int rc = O_OK;
  const int R = 2 * D + 1;
  double *P = (double *)malloc(sizeof(double) * (size_t)(D + 1) * V);
  double *Q = (double *)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1) * V);
  double *w = (double *)malloc(sizeof(double) * (size_t)V);
  double *lv = (double *)malloc(sizeof(double) * (size_t)V);
  int *order = (int *)malloc(sizeof(int) * (size_t)V);
  for (int b = 0; b < B; ++b) {
    const int64_t r0 = (int64_t)b * R;
    for (int i = 0; i <= D; ++i)
      softmax_row(target, dtype, ((int64_t)b * (D + 1) + i) * V, V, temperature, top_p, cut ? cut + r0 + i : NULL,
                  P + (int64_t)i * V, lv, order, cut_used ? cut_used + r0 + i : NULL);
    for (int i = 0; i < D; ++i)
      softmax_row(draftl, dtype, ((int64_t)b * D + i) * V, V, temperature, top_p,
                  cut ? cut + r0 + D + 1 + i : NULL, Q + (int64_t)i * V, lv, order,
                  cut_used ? cut_used + r0 + D + 1 + i : NULL);
    if (sample_row(P, Q, D, V, draft + (int64_t)b * D, u_accept + (int64_t)b * D, u_draw + (int64_t)b * (D + 1),
                   w, &accept_len[b], &next_token[b], mass ? &mass[b] : NULL))
      rc = O_E_PRECOND;
  }
  free(P);
  free(Q);
  free(w);
  free(lv);
  free(order);
  return rc;
}

/* One row's probabilities as softmax_row computes them (for tests: the band
 * rule needs the exact masses the draw compared); `cut` as above, nullable. */
EXPORT int oracle_softmax_row(const void *logits, int dtype, int V, float temperature, float top_p,
                              const float *cut, double *out) {
  if (V <= 0 || !(temperature > 0.0f) || !isfinite(temperature) || !(top_p > 0.0f) || top_p > 1.0f)
    return O_E_ARG;
  double *lv = (double *)malloc(sizeof(double) * (size_t)V);
  int *order = (int *)malloc(sizeof(int) * (size_t)V);
  softmax_row(logits, dtype, 0, V, temperature, top_p, cut, out, lv, order, NULL);
  free(lv);
  free(order);
  return O_OK;
}

/* ------------------------------------------------------------ realignment
 * Buffers: KV [L][2][rows][H][cap][Dh] with esize-byte elements; tokens and
 * position ids int32 [rows][cap]; mask int8 [rows][cap], 1 on content.
 * [BD] 2.1: after each round every row has the same pad + content length
 * (rectangular alignment) and position ids run 0,1,.. over the content as the
 * attention mask marks it (position-id contiguity).  [BD] 2.2 EQSPEC: unpad
 * every row, append its accepted tokens and bonus/replacement token, left-pad
 * all rows to the longest one, recompute the position ids and shift the KV
 * cache to match.  [NL] "Acceptance changes ...": committed KV entries are kept
 * and speculative ones committed or discarded once acceptance is known.
 * Readings: row b commits n = a+1 tokens (its a accepted drafts and the
 * replacement/bonus) and keeps the first n of the D+1 speculative KV entries;
 * the new width is the longest row (tight); pad KV entries are zero bytes, pad
 * tokens are pad_token, pad position ids are 0; only positions [0, width) of
 * the output are written; in and out do not overlap. */

static int row_content_ok(const int8_t *mask, int S, int c) {
  /* a left-padded row of width S with c content tokens: mask = 0^(S-c) 1^c */
  for (int j = 0; j < S; ++j)
    if (mask[j] != (j >= S - c)) return 0;
  return 1;
}

static void positions_from_mask(const int8_t *mask, int W, int32_t *pos) {
  int seen = 0;
  for (int j = 0; j < W; ++j) {
    if (mask[j]) { pos[j] = seen; ++seen; }
    else pos[j] = 0;
  }
}

EXPORT int oracle_realign_eqspec(int L, int H, int Dh, int esize, int B, int cap_in, int cap_out, int D,
                                 const void *kv_in, void *kv_out, const void *kv_new, const int32_t *len_in,
                                 int32_t width_in, const int32_t *tok_in, const int8_t *mask_in,
                                 const int32_t *accept_len, const int32_t *next_token, const int32_t *draft,
                                 int32_t pad_token, int32_t *tok_out, int32_t *pos_out, int8_t *mask_out,
                                 int32_t *len_out, int32_t *width_out) {
  if (L < 0 || H <= 0 || Dh <= 0 || esize <= 0 || B < 0 || D < 0 || width_in < 0 || width_in > cap_in)
    return O_E_ARG;
  const size_t pbytes = (size_t)Dh * (size_t)esize; /* one position of one head */
  const int S = width_in;
  /* step 1 (unpad) and 2 (append) on the token sequences */
  int32_t **content = (int32_t **)calloc((size_t)(B > 0 ? B : 1), sizeof(int32_t *));
  int *clen = (int *)calloc((size_t)(B > 0 ? B : 1), sizeof(int));
  int rc = O_OK, Snew = 0;
  for (int b = 0; b < B && rc == O_OK; ++b) {
    const int c = len_in[b], a = accept_len[b];
    if (c < 0 || c > S || a < 0 || a > D) { rc = O_E_PRECOND; break; }
    if (mask_in && !row_content_ok(mask_in + (size_t)b * cap_in, S, c)) { rc = O_E_PRECOND; break; }
    content[b] = (int32_t *)malloc(sizeof(int32_t) * (size_t)(c + a + 1));
    int k = 0;
    for (int j = S - c; j < S; ++j) content[b][k++] = tok_in[(size_t)b * cap_in + j];  /* unpad */
    for (int i = 0; i < a; ++i) content[b][k++] = draft[(size_t)b * D + i];           /* accepted drafts */
    content[b][k++] = next_token[b];                                                   /* replacement/bonus */
    clen[b] = k;
    if (k > Snew) Snew = k;
  }
  if (rc == O_OK && Snew > cap_out) rc = O_E_CAPACITY;
  if (rc != O_OK) {
    for (int b = 0; b < B; ++b) free(content[b]);
    free(content); free(clen);
    return rc;
  }
  /* step 3 (repad): left-pad to the longest row, mask, positions from the mask */
  for (int b = 0; b < B; ++b) {
    const int pad = Snew - clen[b];
    int8_t *m = mask_out + (size_t)b * cap_out;
    for (int j = 0; j < Snew; ++j) {
      m[j] = (int8_t)(j >= pad);
      tok_out[(size_t)b * cap_out + j] = (j >= pad) ? content[b][j - pad] : pad_token;
    }
    positions_from_mask(m, Snew, pos_out + (size_t)b * cap_out);
    len_out[b] = clen[b];
  }
  *width_out = Snew;
  /* the same unpad / append / repad on every (layer, K|V, head) KV sequence */
#pragma omp parallel
  {
  unsigned char *tmp = (unsigned char *)malloc(pbytes * (size_t)(cap_in + D + 1));
#pragma omp for collapse(4) schedule(static)
  for (int l = 0; l < L; ++l)
    for (int kv = 0; kv < 2; ++kv)
      for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
          const size_t seg_in = ((((size_t)l * 2 + kv) * B + b) * H + h) * (size_t)cap_in * pbytes;
          const size_t seg_out = ((((size_t)l * 2 + kv) * B + b) * H + h) * (size_t)cap_out * pbytes;
          const size_t seg_new = ((((size_t)l * 2 + kv) * B + b) * H + h) * (size_t)(D + 1) * pbytes;
          const int c = len_in[b], n = accept_len[b] + 1, pad = Snew - clen[b];
          size_t k = 0;
          for (int j = S - c; j < S; ++j, ++k)
            memcpy(tmp + k * pbytes, (const unsigned char *)kv_in + seg_in + (size_t)j * pbytes, pbytes);
          for (int j = 0; j < n; ++j, ++k)
            memcpy(tmp + k * pbytes, (const unsigned char *)kv_new + seg_new + (size_t)j * pbytes, pbytes);
          unsigned char *dst = (unsigned char *)kv_out + seg_out;
          memset(dst, 0, (size_t)pad * pbytes);
          memcpy(dst + (size_t)pad * pbytes, tmp, k * pbytes);
        }
  free(tmp);
  }
  for (int b = 0; b < B; ++b) free(content[b]);
  free(content); free(clen);
  return O_OK;
}

/* ------------------------------------------------------- EXSPEC grouping
 * [BD] 2.3: keep a pool of active sequences rather than a fixed batch, group
 * sequences of equal length into batches, which then need no realignment, and
 * realign only mixed-length batches.
 * Reading (one admissible policy, fixed so results are comparable): order the
 * ids by (length, id); for each length in ascending order emit floor(cnt/G)
 * full batches of that length; then chunk the remaining ids, still in (length,
 * id) order, into batches of G (the last may be short).  For every batch:
 * uniform = all its lengths equal, width = its longest length.  n_uniform is
 * the number of uniform batches. */
static const int32_t *g_len_for_sort;
static int cmp_len_id(const void *x, const void *y) {
  const int32_t i = *(const int32_t *)x, j = *(const int32_t *)y;
  if (g_len_for_sort[i] != g_len_for_sort[j]) return g_len_for_sort[i] < g_len_for_sort[j] ? -1 : 1;
  return (i > j) - (i < j);
}

EXPORT int oracle_group_by_len(const int32_t *len, int N, int G, int32_t *order, int32_t *uniform,
                               int32_t *width, int32_t *n_uniform) {
  if (N < 0 || G <= 0) return O_E_ARG;
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  for (int i = 0; i < N; ++i) ids[i] = i;
  g_len_for_sort = len;
  qsort(ids, (size_t)N, sizeof(int32_t), cmp_len_id);
  int out = 0;
  int32_t *left = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  int nleft = 0;
  for (int s = 0; s < N;) {
    int e = s;
    while (e < N && len[ids[e]] == len[ids[s]]) ++e;
    const int full = ((e - s) / G) * G;
    for (int k = s; k < s + full; ++k) order[out++] = ids[k];
    for (int k = s + full; k < e; ++k) left[nleft++] = ids[k];
    s = e;
  }
  for (int k = 0; k < nleft; ++k) order[out++] = left[k];
  const int nb = (N + G - 1) / G;
  int nu = 0;
  for (int g = 0; g < nb; ++g) {
    const int lo = g * G, hi = (lo + G < N) ? lo + G : N;
    int mn = len[order[lo]], mx = len[order[lo]];
    for (int k = lo; k < hi; ++k) {
      if (len[order[k]] < mn) mn = len[order[k]];
      if (len[order[k]] > mx) mx = len[order[k]];
    }
    uniform[g] = (mn == mx);
    width[g] = mx;
    nu += (mn == mx);
  }
  *n_uniform = nu;
  free(ids);
  free(left);
  return O_OK;
}

/* ----------------------------------------------- EXSPEC gather / append
 * Reading of [BD] 2.3 for storage: pool rows hold their content left-aligned
 * from position 0 with no padding, so a same-length batch is already
 * rectangular with position ids 0..len-1 and is not copied.  A mixed batch is
 * realigned into a left-padded rectangle of width = its longest row (the same
 * repad as EQSPEC, without an append).  After verification every sequence
 * appends its committed tokens and KV entries in place at its length. */
EXPORT int oracle_gather(int L, int H, int Dh, int esize, int N, int cap_pool, const void *kv_pool,
                         const int32_t *tok_pool, const int32_t *len_pool, const int32_t *rows, int B, int G,
                         const int32_t *skip_group, int cap_out, void *kv_out, int32_t *tok_out, int32_t *pos_out,
                         int8_t *mask_out, int32_t *width_out, int32_t pad_token) {
  if (L < 0 || H <= 0 || Dh <= 0 || esize <= 0 || B < 0 || G <= 0) return O_E_ARG;
  const size_t pbytes = (size_t)Dh * (size_t)esize;
  const int ng = (B + G - 1) / G;
  for (int g = 0; g < ng; ++g) {
    if (skip_group && skip_group[g]) continue;
    const int lo = g * G, hi = (lo + G < B) ? lo + G : B;
    int W = 0;
    for (int j = lo; j < hi; ++j) {
      const int r = rows ? rows[j] : j;
      if (r < 0 || r >= N || len_pool[r] < 0 || len_pool[r] > cap_pool) return O_E_PRECOND;
      if (len_pool[r] > W) W = len_pool[r];
    }
    if (W > cap_out) return O_E_CAPACITY;
    width_out[g] = W;
    for (int j = lo; j < hi; ++j) {
      const int r = rows ? rows[j] : j, c = len_pool[r], pad = W - c;
      int8_t *m = mask_out + (size_t)j * cap_out;
      for (int x = 0; x < W; ++x) {
        m[x] = (int8_t)(x >= pad);
        tok_out[(size_t)j * cap_out + x] = (x >= pad) ? tok_pool[(size_t)r * cap_pool + (x - pad)] : pad_token;
      }
      positions_from_mask(m, W, pos_out + (size_t)j * cap_out);
      for (int l = 0; l < L; ++l)
        for (int kv = 0; kv < 2; ++kv)
          for (int h = 0; h < H; ++h) {
            const unsigned char *src = (const unsigned char *)kv_pool +
                                       ((((size_t)l * 2 + kv) * N + r) * H + h) * (size_t)cap_pool * pbytes;
            unsigned char *dst = (unsigned char *)kv_out +
                                 ((((size_t)l * 2 + kv) * B + j) * H + h) * (size_t)cap_out * pbytes;
            memset(dst, 0, (size_t)pad * pbytes);
            memcpy(dst + (size_t)pad * pbytes, src, (size_t)c * pbytes);
          }
    }
  }
  return O_OK;
}

EXPORT int oracle_append(int L, int H, int Dh, int esize, int N, int cap_pool, void *kv_pool, int32_t *tok_pool,
                         int32_t *len_pool, const int32_t *rows, int B, int D, const void *kv_new,
                         const int32_t *draft, const int32_t *accept_len, const int32_t *next_token) {
  if (L < 0 || H <= 0 || Dh <= 0 || esize <= 0 || B < 0 || D < 0) return O_E_ARG;
  const size_t pbytes = (size_t)Dh * (size_t)esize;
  unsigned char *seen = (unsigned char *)calloc((size_t)(N > 0 ? N : 1), 1);
  int rc = O_OK;
  for (int b = 0; b < B && rc == O_OK; ++b) {
    const int r = rows ? rows[b] : b;
    if (r < 0 || r >= N || seen[r] || accept_len[b] < 0 || accept_len[b] > D || len_pool[r] < 0) rc = O_E_PRECOND;
    else if (len_pool[r] + accept_len[b] + 1 > cap_pool) rc = O_E_CAPACITY;
    else seen[r] = 1;
  }
  free(seen);
  if (rc != O_OK) return rc;
  for (int b = 0; b < B; ++b) {
    const int r = rows ? rows[b] : b, c = len_pool[r], a = accept_len[b], n = a + 1;
    if (tok_pool) {
      for (int i = 0; i < a; ++i) tok_pool[(size_t)r * cap_pool + c + i] = draft[(size_t)b * D + i];
      tok_pool[(size_t)r * cap_pool + c + a] = next_token[b];
    }
    for (int l = 0; l < L; ++l)
      for (int kv = 0; kv < 2; ++kv)
        for (int h = 0; h < H; ++h) {
          unsigned char *dst = (unsigned char *)kv_pool +
                               ((((size_t)l * 2 + kv) * N + r) * H + h) * (size_t)cap_pool * pbytes;
          const unsigned char *src = (const unsigned char *)kv_new +
                                     ((((size_t)l * 2 + kv) * B + b) * H + h) * (size_t)(D + 1) * pbytes;
          memcpy(dst + (size_t)c * pbytes, src, (size_t)n * pbytes);
        }
    len_pool[r] = c + n;
  }
  return O_OK;
}

/* ------------------------------------------------------------ paged KV
 * [AB] ties the superlinear cost of realignment to contiguous cache layouts.
 * With a block table the cache is a pool of pages of `page` positions, and a
 * row's content position j lives in page bt[row][j / page], slot j % page:
 *   pages       [L][2][n_pages][H][page][Dh], esize-byte elements;
 *   bt          int32 [rows][max_blocks], -1 where a row has no page;
 *   free_pages  int32 [n_pages], a stack whose entries [0, *n_free) are free;
 *   tokens      int32 [rows][max_blocks * page], each row's content from 0;
 *   len         int32 [rows].
 * The rectangle of [BD] 2.1 (every row left-padded to the longest) is then a
 * matter of metadata: row b's pad is S' - len'_b, its position ids run 0.. over
 * the content.  So EQSPEC's unpad-append-repad ([BD] 2.2) reduces to
 * appending each row's committed entries and tokens at its length; the KV
 * already in place never moves.  A gather turns any batch of rows back into the
 * left-padded rectangle EQSPEC would produce.
 * Page allocation (one admissible policy, fixed so that results compare byte
 * for byte; any policy that gives each row distinct free pages is correct):
 * batch entries in order take their new pages from the top of the free stack,
 * the entry's first new block getting the topmost remaining page.  Retiring
 * pushes a row's pages back in block order, entries in batch order.
 * geo = {L, H, Dh, esize, n_pages, page, max_blocks, rows}. */
enum { G_L, G_H, G_DH, G_ES, G_NP, G_PAGE, G_MB, G_ROWS };

static int blocks_for(int n, int page) { return (n + page - 1) / page; }

/* byte offset of (layer l, K|V kv, page pg, head h, slot s) in the page pool */
static size_t page_off(const int32_t *geo, int l, int kv, int pg, int h, int s) {
  const size_t pbytes = (size_t)geo[G_DH] * (size_t)geo[G_ES];
  return (((((size_t)l * 2 + kv) * geo[G_NP] + pg) * geo[G_H] + h) * geo[G_PAGE] + s) * pbytes;
}

static int paged_geo_ok(const int32_t *geo) {
  return geo[G_L] >= 0 && geo[G_H] > 0 && geo[G_DH] > 0 && geo[G_ES] > 0 && geo[G_NP] >= 0 && geo[G_PAGE] > 0 &&
         geo[G_MB] > 0 && geo[G_ROWS] > 0;
}

static int batch_rows_ok(const int32_t *geo, const int32_t *rows, int B) {
  for (int b = 0; b < B; ++b) {
    const int r = rows ? rows[b] : b;
    if (r < 0 || r >= geo[G_ROWS]) return 0;
    for (int o = 0; o < b; ++o)
      if ((rows ? rows[o] : o) == r) return 0;
  }
  return 1;
}

/* One round's realignment on a paged cache: batch entry b (pool row rows[b],
 * NULL = b) commits n_b = accept_len[b] + 1 tokens (its accepted drafts, then
 * next_token[b]) and the first n_b of its D+1 speculative KV entries kv_new
 * [L][2][B][H][D+1][Dh], written at positions len, len+1, ... of the row;
 * new pages come from the free stack as stated above.  *width = S' =
 * max_b(len_b + n_b).  The rectangle view (nullable rect_* [B][rect_cap]):
 * row b left-padded by S' - len'_b with pad_token, position id 0 and mask 0,
 * then its content with position ids 0.. and mask 1.  Errors (nothing
 * written): O_E_ARG for bad geometry, rows or accepted lengths outside [0, D];
 * O_E_CAPACITY when a row would exceed max_blocks * page positions, the batch
 * needs more pages than are free, or S' exceeds rect_cap. */
EXPORT int oracle_paged_append(const int32_t *geo, void *pages, int32_t *bt, int32_t *free_pages, int32_t *n_free,
                               int32_t *tokens, int32_t *len, const int32_t *rows, int B, int D,
                               const void *kv_new, const int32_t *draft, const int32_t *accept_len,
                               const int32_t *next_token, int32_t pad_token, int32_t *width, int32_t *rect_tok,
                               int32_t *rect_pos, int8_t *rect_mask, int rect_cap) {
  if (!paged_geo_ok(geo) || B < 0 || D < 0 || !batch_rows_ok(geo, rows, B)) return O_E_ARG;
  const int page = geo[G_PAGE], tcap = geo[G_MB] * page;
  const size_t pbytes = (size_t)geo[G_DH] * (size_t)geo[G_ES];
  int Snew = 0, need = 0;
  for (int b = 0; b < B; ++b) {
    const int r = rows ? rows[b] : b, c = len[r], a = accept_len[b];
    if (a < 0 || a > D || c < 0 || c > tcap) return O_E_ARG;
    const int cn = c + a + 1;
    if (cn > tcap) return O_E_CAPACITY;
    need += blocks_for(cn, page) - blocks_for(c, page);
    if (cn > Snew) Snew = cn;
  }
  if (need > *n_free || (rect_tok && Snew > rect_cap)) return O_E_CAPACITY;
  /* pages: pop from the top of the free stack, batch entries in order */
  int top = *n_free;
  for (int b = 0; b < B; ++b) {
    const int r = rows ? rows[b] : b, c = len[r], cn = c + accept_len[b] + 1;
    for (int blk = blocks_for(c, page); blk < blocks_for(cn, page); ++blk) bt[(size_t)r * geo[G_MB] + blk] =
        free_pages[--top];
  }
  *n_free = top;
  /* committed KV entries and tokens at the row's end */
  for (int b = 0; b < B; ++b) {
    const int r = rows ? rows[b] : b, c = len[r], a = accept_len[b], n = a + 1;
    for (int l = 0; l < geo[G_L]; ++l)
      for (int kv = 0; kv < 2; ++kv)
        for (int h = 0; h < geo[G_H]; ++h)
          for (int i = 0; i < n; ++i) {
            const int j = c + i, pg = bt[(size_t)r * geo[G_MB] + j / page];
            const size_t src = (((((size_t)l * 2 + kv) * B + b) * geo[G_H] + h) * (size_t)(D + 1) + i) * pbytes;
            memcpy((unsigned char *)pages + page_off(geo, l, kv, pg, h, j % page),
                   (const unsigned char *)kv_new + src, pbytes);
          }
    int32_t *t = tokens + (size_t)r * tcap + c;
    for (int i = 0; i < a; ++i) t[i] = draft[(size_t)b * D + i];
    t[a] = next_token[b];
    len[r] = c + n;
  }
  *width = Snew;
  /* the rectangle view of the batch: [BD] 2.1's alignment as metadata */
  if (rect_tok)
    for (int b = 0; b < B; ++b) {
      const int r = rows ? rows[b] : b, pad = Snew - len[r];
      for (int j = 0; j < Snew; ++j) {
        const int in = j >= pad;
        rect_tok[(size_t)b * rect_cap + j] = in ? tokens[(size_t)r * tcap + j - pad] : pad_token;
        if (rect_mask) rect_mask[(size_t)b * rect_cap + j] = (int8_t)in;
      }
      if (rect_pos) {
        int8_t *m = (int8_t *)malloc((size_t)(Snew > 0 ? Snew : 1));
        for (int j = 0; j < Snew; ++j) m[j] = (int8_t)(j >= pad);
        positions_from_mask(m, Snew, rect_pos + (size_t)b * rect_cap);
        free(m);
      }
    }
  return O_OK;
}

/* The batch's rows as the left-padded rectangle of width W = their longest
 * length: out_kv [L][2][B][H][cap_out][Dh] (zero bytes on the pad), tokens,
 * position ids and mask [B][cap_out], out_len [B] and *width = W; positions
 * [W, cap_out) are not written.  O_E_CAPACITY if W > cap_out. */
EXPORT int oracle_paged_gather(const int32_t *geo, const void *pages, const int32_t *bt, const int32_t *tokens,
                               const int32_t *len, const int32_t *rows, int B, int cap_out, void *out_kv,
                               int32_t *out_tok, int32_t *out_pos, int8_t *out_mask, int32_t *out_len,
                               int32_t *width, int32_t pad_token) {
  if (!paged_geo_ok(geo) || B < 0 || !batch_rows_ok(geo, rows, B)) return O_E_ARG;
  const int page = geo[G_PAGE], tcap = geo[G_MB] * page;
  const size_t pbytes = (size_t)geo[G_DH] * (size_t)geo[G_ES];
  int W = 0;
  for (int b = 0; b < B; ++b) {
    const int c = len[rows ? rows[b] : b];
    if (c < 0 || c > tcap) return O_E_ARG;
    if (c > W) W = c;
  }
  if (W > cap_out) return O_E_CAPACITY;
  for (int b = 0; b < B; ++b) {
    const int r = rows ? rows[b] : b, c = len[r], pad = W - c;
    for (int l = 0; l < geo[G_L]; ++l)
      for (int kv = 0; kv < 2; ++kv)
        for (int h = 0; h < geo[G_H]; ++h) {
          unsigned char *dst =
              (unsigned char *)out_kv + ((((size_t)l * 2 + kv) * B + b) * geo[G_H] + h) * (size_t)cap_out * pbytes;
          memset(dst, 0, (size_t)pad * pbytes);
          for (int j = 0; j < c; ++j)
            memcpy(dst + (size_t)(pad + j) * pbytes,
                   (const unsigned char *)pages + page_off(geo, l, kv, bt[(size_t)r * geo[G_MB] + j / page], h,
                                                           j % page),
                   pbytes);
        }
    int8_t *m = out_mask + (size_t)b * cap_out;
    for (int j = 0; j < W; ++j) {
      m[j] = (int8_t)(j >= pad);
      out_tok[(size_t)b * cap_out + j] = j >= pad ? tokens[(size_t)r * tcap + j - pad] : pad_token;
    }
    positions_from_mask(m, W, out_pos + (size_t)b * cap_out);
    out_len[b] = c;
  }
  *width = W;
  return O_OK;
}

/* Admit: batch entry b's content, positions [S - in_len[b], S) of a
 * left-padded rectangle in_kv [L][2][B][H][cap_in][Dh] with tokens
 * in_tok [B][cap_in] (a prefill's output), becomes pool row rows[b], which
 * must be empty (length 0, no pages).  Pages come from the free stack as for
 * append.  Errors (nothing written): O_E_ARG (geometry, rows, a non-empty row,
 * lengths outside [0, S], S > cap_in), O_E_CAPACITY (too few free pages or
 * positions). */
EXPORT int oracle_paged_admit(const int32_t *geo, void *pages, int32_t *bt, int32_t *free_pages, int32_t *n_free,
                              int32_t *tokens, int32_t *len, const int32_t *rows, int B, const void *in_kv,
                              const int32_t *in_tok, const int32_t *in_len, int S, int cap_in) {
  if (!paged_geo_ok(geo) || B < 0 || S < 0 || S > cap_in || !batch_rows_ok(geo, rows, B)) return O_E_ARG;
  const int page = geo[G_PAGE], tcap = geo[G_MB] * page;
  const size_t pbytes = (size_t)geo[G_DH] * (size_t)geo[G_ES];
  int need = 0;
  for (int b = 0; b < B; ++b) {
    const int r = rows ? rows[b] : b, c = in_len[b];
    if (len[r] != 0 || c < 0 || c > S) return O_E_ARG;
    if (c > tcap) return O_E_CAPACITY;
    need += blocks_for(c, page);
  }
  if (need > *n_free) return O_E_CAPACITY;
  int top = *n_free;
  for (int b = 0; b < B; ++b) {
    const int r = rows ? rows[b] : b, c = in_len[b];
    for (int blk = 0; blk < blocks_for(c, page); ++blk) bt[(size_t)r * geo[G_MB] + blk] = free_pages[--top];
    for (int l = 0; l < geo[G_L]; ++l)
      for (int kv = 0; kv < 2; ++kv)
        for (int h = 0; h < geo[G_H]; ++h) {
          const unsigned char *src = (const unsigned char *)in_kv +
                                     ((((size_t)l * 2 + kv) * B + b) * geo[G_H] + h) * (size_t)cap_in * pbytes;
          for (int j = 0; j < c; ++j)
            memcpy((unsigned char *)pages + page_off(geo, l, kv, bt[(size_t)r * geo[G_MB] + j / page], h, j % page),
                   src + (size_t)(S - c + j) * pbytes, pbytes);
        }
    for (int j = 0; j < c; ++j) tokens[(size_t)r * tcap + j] = in_tok[(size_t)b * cap_in + S - c + j];
    len[r] = c;
  }
  *n_free = top;
  return O_OK;
}

/* Retire: the batch's rows give their pages back (pushed on the free stack in
 * block order, entries in batch order), their block-table entries become -1
 * and their lengths 0.  O_E_ARG for bad rows or lengths. */
EXPORT int oracle_paged_retire(const int32_t *geo, int32_t *bt, int32_t *free_pages, int32_t *n_free, int32_t *len,
                               const int32_t *rows, int B) {
  if (!paged_geo_ok(geo) || B < 0 || !batch_rows_ok(geo, rows, B)) return O_E_ARG;
  const int page = geo[G_PAGE], tcap = geo[G_MB] * page;
  for (int b = 0; b < B; ++b) {
    const int c = len[rows ? rows[b] : b];
    if (c < 0 || c > tcap) return O_E_ARG;
  }
  int top = *n_free, back = 0;
  for (int b = 0; b < B; ++b) back += blocks_for(len[rows ? rows[b] : b], page);
  if (top < 0 || top + back > geo[G_NP]) return O_E_ARG; /* more pages than exist: a corrupt table */
  for (int b = 0; b < B; ++b) {
    const int r = rows ? rows[b] : b;
    for (int blk = 0; blk < blocks_for(len[r], page); ++blk) {
      free_pages[top++] = bt[(size_t)r * geo[G_MB] + blk];
      bt[(size_t)r * geo[G_MB] + blk] = -1;
    }
    len[r] = 0;
  }
  *n_free = top;
  return O_OK;
}

/* ------------------------------------------------------- pool lifecycle
 * [BD] 2.3: EXSPEC keeps a pool of active sequences rather than a fixed batch
 * and regroups them every round; sequences leave the pool when they finish and
 * new ones join it.  The pages name the pool but not its policies; one
 * admissible set is fixed here so results compare byte for byte:
 *  - schedule: every active sequence runs every round; `active` lists their
 *    pool slots in schedule order;
 *  - finish: after a round's append, a sequence finishes at the first newly
 *    committed position p holding the end-of-sequence id, or with p + 1 >=
 *    max_len; its length becomes p + 1 (later committed entries are dropped),
 *    it leaves the active list (the others keep their order) and its slot
 *    joins the free slots, which are kept in ascending order;
 *  - admit: queued prompts are taken in queue order, each into the lowest free
 *    slot, and join the end of the active list; a prompt's content (positions
 *    [0, plen) of the queue's own left-aligned buffer) and token ids are copied
 *    into the slot.
 * The pool is left-aligned: slot s holds its content at positions [0, len[s]). */

/* rows [B] is the round's batch order over the active slots (B == *n_active)
 * and accept_len its accepted lengths; the append has already run.  Writes
 * retired [*n_retired] (finished slots in active-list order) and updates len,
 * active, free_slots.  O_E_ARG: rows not a permutation of the active list,
 * accepted lengths outside [0, D], a length shorter than its committed
 * tokens, or max_len < 1. */
EXPORT int oracle_pool_finish(const int32_t *tok_pool, int cap_pool, int32_t *len_pool, int slots, int32_t *active,
                              int32_t *n_active, int32_t *free_slots, int32_t *n_free, const int32_t *rows,
                              const int32_t *accept_len, int B, int D, int32_t eos_id, int32_t max_len,
                              int32_t *retired, int32_t *n_retired) {
  if (slots < 1 || B != *n_active || B < 0 || B > slots || max_len < 1 || D < 0) return O_E_ARG;
  int32_t *in_batch = (int32_t *)calloc((size_t)slots, sizeof(int32_t));
  int32_t *newlen = (int32_t *)malloc(sizeof(int32_t) * (size_t)slots);
  int rc = O_OK;
  for (int j = 0; j < B && rc == O_OK; ++j) {
    const int s = rows[j], a = accept_len[j];
    if (s < 0 || s >= slots || in_batch[s] || a < 0 || a > D) { rc = O_E_ARG; break; }
    in_batch[s] = 1;
    const int cn = len_pool[s], c = cn - (a + 1);
    if (c < 0 || cn > cap_pool) { rc = O_E_ARG; break; }
    newlen[s] = -1;
    for (int p = c; p < cn; ++p)
      if (tok_pool[(size_t)s * cap_pool + p] == eos_id || p + 1 >= max_len) { newlen[s] = p + 1; break; }
  }
  for (int j = 0; j < B && rc == O_OK; ++j)
    if (active[j] < 0 || active[j] >= slots || !in_batch[active[j]]) rc = O_E_ARG;
  if (rc != O_OK) { free(in_batch); free(newlen); return rc; }
  int na = 0, nr = 0;
  int32_t *is_free = (int32_t *)calloc((size_t)slots, sizeof(int32_t));
  for (int i = 0; i < *n_free; ++i) is_free[free_slots[i]] = 1;
  for (int j = 0; j < B; ++j) {
    const int s = active[j];
    if (newlen[s] >= 0) {
      len_pool[s] = newlen[s];
      retired[nr++] = s;
      is_free[s] = 1;
    } else {
      active[na++] = s;
    }
  }
  int nf = 0;
  for (int s = 0; s < slots; ++s)
    if (is_free[s]) free_slots[nf++] = s;
  *n_active = na;
  *n_free = nf;
  *n_retired = nr;
  free(in_batch); free(newlen); free(is_free);
  return O_OK;
}

/* Admit from the queue: prompts [*q_head, Q) of pkv [L][2][Q][H][pcap][Dh],
 * ptok [Q][pcap], plen [Q], as many as there are free slots.  Writes admitted
 * [*n_admitted] (slots, in admission order).  O_E_CAPACITY (nothing written)
 * if an admitted prompt is longer than the pool's cap; O_E_ARG for lengths
 * outside [0, pcap]. */
EXPORT int oracle_pool_admit(int L, int H, int Dh, int esize, void *kv_pool, int32_t *tok_pool, int cap_pool,
                             int32_t *len_pool, int slots, int32_t *active, int32_t *n_active, int32_t *free_slots,
                             int32_t *n_free, int32_t *q_head, int Q, const void *pkv, const int32_t *ptok,
                             const int32_t *plen, int pcap, int32_t *admitted, int32_t *n_admitted) {
  if (L < 0 || H <= 0 || Dh <= 0 || esize <= 0 || slots < 1 || Q < 0 || *q_head < 0 || *q_head > Q) return O_E_ARG;
  const size_t pbytes = (size_t)Dh * (size_t)esize;
  int k = *n_free < Q - *q_head ? *n_free : Q - *q_head;
  for (int i = 0; i < k; ++i) {
    const int q = *q_head + i;
    if (plen[q] < 0 || plen[q] > pcap) return O_E_ARG;
    if (plen[q] > cap_pool) return O_E_CAPACITY;
  }
  for (int i = 0; i < k; ++i) {
    const int s = free_slots[i], q = *q_head + i, n = plen[q];
    for (int l = 0; l < L; ++l)
      for (int kv = 0; kv < 2; ++kv)
        for (int h = 0; h < H; ++h) {
          const unsigned char *src =
              (const unsigned char *)pkv + ((((size_t)l * 2 + kv) * Q + q) * H + h) * (size_t)pcap * pbytes;
          unsigned char *dst =
              (unsigned char *)kv_pool + ((((size_t)l * 2 + kv) * slots + s) * H + h) * (size_t)cap_pool * pbytes;
          memcpy(dst, src, (size_t)n * pbytes);
        }
    for (int j = 0; j < n; ++j) tok_pool[(size_t)s * cap_pool + j] = ptok[(size_t)q * pcap + j];
    len_pool[s] = n;
    active[*n_active + i] = s;
    admitted[i] = s;
  }
  for (int i = k; i < *n_free; ++i) free_slots[i - k] = free_slots[i];
  *n_free -= k;
  *n_active += k;
  *q_head += k;
  *n_admitted = k;
  return O_OK;
}
