// C ABI of libspecdec: host-side validation, then one stream-ordered launch
// per step.  Declarations and the contract of every entry point are in
// include/specdec.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "launch.h"
#include "specdec.h"

#define EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxPool = 4096;

size_t esize(int dtype) { return dtype == SPECDEC_F32 ? 4 : 2; }
bool dtype_ok(int dtype) { return dtype == SPECDEC_F32 || dtype == SPECDEC_F16 || dtype == SPECDEC_BF16; }
hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }
int launched(hipError_t e) { return e == hipSuccess ? SPECDEC_OK : SPECDEC_E_LAUNCH; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t kv_bytes(const specdec_seqbuf_t *s) {
  return (size_t)s->layers * 2 * (size_t)s->rows * (size_t)s->heads * (size_t)s->cap * (size_t)s->head_dim *
         esize(s->dtype);
}

// greedy workspace: one atomic line per key and per batch-row counter
size_t ws_keys_bytes(int B, int D) { return (size_t)B * ((size_t)D + 1) * sd::kAtomicLine; }

int check_seqbuf_shape(const specdec_seqbuf_t *s) {
  if (!s) return SPECDEC_E_ARG;
  if (s->rows < 0 || s->cap < 0 || s->layers < 0 || s->heads < 1 || s->head_dim < 1) return SPECDEC_E_ARG;
  if (!dtype_ok(s->dtype)) return SPECDEC_E_DTYPE;
  // an empty buffer may come without an address (a zero-size tensor has none)
  if ((!s->kv && kv_bytes(s) > 0) || (!s->len && s->rows > 0)) return SPECDEC_E_ARG;
  if (((size_t)s->head_dim * esize(s->dtype)) % 16 != 0) return SPECDEC_E_ALIGN;
  if (reinterpret_cast<uintptr_t>(s->kv) % 16 != 0) return SPECDEC_E_ALIGN;
  return SPECDEC_OK;
}

bool same_geometry(const specdec_seqbuf_t *a, const specdec_seqbuf_t *b) {
  return a->layers == b->layers && a->heads == b->heads && a->head_dim == b->head_dim && a->dtype == b->dtype;
}

// the two descriptors name the same buffers with the same shape
bool same_buffers(const specdec_seqbuf_t *a, const specdec_seqbuf_t *b) {
  return a->kv == b->kv && a->tokens == b->tokens && a->pos == b->pos && a->mask == b->mask && a->len == b->len &&
         a->width == b->width && a->rows == b->rows && a->cap == b->cap && same_geometry(a, b);
}

}  // namespace

EXPORT const char *specdec_version(void) { return "specdec 0.1 gfx950"; }


EXPORT size_t specdec_workspace_bytes(int B, int D) {
  // 0 for sizes specdec_verify_greedy rejects anyway (and whose byte count
  // could wrap)
  if (B < 0 || D < 0 || D > 255 || (long long)B * ((long long)D + 1) > (1LL << 24)) return 0;
  return ws_keys_bytes(B, D) + (size_t)B * sd::kAtomicLine;
}

EXPORT int specdec_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (!ws) return SPECDEC_E_WORKSPACE;
  return launched(sd::launch_zero(ws, ws_bytes / 4 * 4, as_stream(stream)));
}

EXPORT int specdec_verify_greedy(const void *logits, int dtype, int64_t row_stride, int B, int D, int V,
                                 const int32_t *draft, int32_t *accept_len, int32_t *next_token,
                                 int32_t *target_tok, void *ws, size_t ws_bytes, int32_t *status, void *stream) {
  if (B < 0 || D < 0 || V < 1 || row_stride < V) return SPECDEC_E_ARG;
  if (!dtype_ok(dtype)) return SPECDEC_E_DTYPE;
  if (B == 0) return SPECDEC_OK;
  if (!logits || !accept_len || !next_token || (D > 0 && !draft)) return SPECDEC_E_ARG;
  if (D > 255 || (long long)B * ((long long)D + 1) > (1LL << 24) || (long long)V > (1LL << 30)) return SPECDEC_E_ARG;
  if (!ws || ws_bytes < specdec_workspace_bytes(B, D) || reinterpret_cast<uintptr_t>(ws) % 8 != 0)
    return SPECDEC_E_WORKSPACE;
  sd::GreedyParams p;
  p.logits = logits;
  p.dtype = dtype;
  p.row_stride = row_stride;
  p.B = B;
  p.D = D;
  p.V = V;
  p.draft = draft;
  p.accept_len = accept_len;
  p.next_token = next_token;
  p.target_tok = target_tok;
  p.keys = static_cast<unsigned long long *>(ws);
  p.counters = reinterpret_cast<unsigned int *>(static_cast<char *>(ws) + ws_keys_bytes(B, D));
  p.status = status;
  p.vec = reinterpret_cast<uintptr_t>(logits) % 16 == 0 && ((size_t)row_stride * esize(dtype)) % 16 == 0;
  return launched(sd::launch_verify_greedy(p, as_stream(stream)));
}

EXPORT int specdec_verify_greedy_noalloc(const void *logits, int dtype, int64_t row_stride, int B, int D, int V,
                                         const int32_t *draft, int32_t *accept_len, int32_t *next_token,
                                         int32_t *target_tok, int32_t *status, void *stream) {
  // the argument checks of specdec_verify_greedy come first, so both calls
  // reject the same arguments the same way; the size limit needs no HIP call
  if (B < 0 || D < 0 || V < 1 || row_stride < V) return SPECDEC_E_ARG;
  if (!dtype_ok(dtype)) return SPECDEC_E_DTYPE;
  if (B == 0) return SPECDEC_OK;
  if (!logits || !accept_len || !next_token || (D > 0 && !draft)) return SPECDEC_E_ARG;
  if (D > 255 || (long long)B * ((long long)D + 1) > (1LL << 24) || (long long)V > (1LL << 30)) return SPECDEC_E_ARG;
  if (specdec_workspace_bytes(B, D) > SPECDEC_STATIC_SCRATCH_BYTES) return SPECDEC_E_SCRATCH;
  void *ws = nullptr;
  if (sd::static_scratch(&ws, as_stream(stream)) != hipSuccess) return SPECDEC_E_LAUNCH;
  return specdec_verify_greedy(logits, dtype, row_stride, B, D, V, draft, accept_len, next_token, target_tok, ws,
                               SPECDEC_STATIC_SCRATCH_BYTES, status, stream);
}

// sampled verification's workspace: a fixed-size block per batch row (a
// counter line and the row's run masses), so one workspace serves any later
// call with as many rows or fewer, whatever its D and V
EXPORT size_t specdec_verify_sample_workspace_bytes(int B, int D, int V) {
  if (B < 0 || D < 0 || V < 1 || (long long)B > (1LL << 30) || (long long)V > (1LL << 30)) return 0;
  return (size_t)B * sd::kSampleRowBytes;
}

EXPORT int specdec_verify_sample(const float *p, const float *q, int B, int D, int V, const int32_t *draft,
                                 const float *u_accept, const float *u_draw, int32_t *accept_len,
                                 int32_t *next_token, void *ws, size_t ws_bytes, int32_t *status, void *stream) {
  if (B < 0 || D < 0 || D > 255 || V < 1) return SPECDEC_E_ARG;
  if (B == 0) return SPECDEC_OK;
  if (!p || !u_draw || !accept_len || !next_token || (D > 0 && (!q || !draft || !u_accept))) return SPECDEC_E_ARG;
  if ((long long)B > (1LL << 30) || (long long)V > (1LL << 30)) return SPECDEC_E_ARG;
  const size_t need = specdec_verify_sample_workspace_bytes(B, D, V);
  if (need == 0) return SPECDEC_E_ARG;
  if (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 16 != 0) return SPECDEC_E_WORKSPACE;
  sd::SampleParams s;
  s.p = p;
  s.q = q;
  s.B = B;
  s.D = D;
  s.V = V;
  sd::sample_shape(V, s.R, s.S);
  s.draft = draft;
  s.u_accept = u_accept;
  s.u_draw = u_draw;
  s.accept_len = accept_len;
  s.next_token = next_token;
  s.status = status;
  if ((long long)B * s.S >= (1LL << 31)) return SPECDEC_E_ARG;
  s.ws = static_cast<char *>(ws);
  return launched(sd::launch_verify_sample(s, as_stream(stream)));
}

// Workspace of specdec_verify_sample_logits: per-split row statistics, the
// logits at the draft tokens, the stop row's per-split and per-run masses, the
// stop row's parameters and the nucleus of every row.
struct SlLayout {
  size_t stats, gath, part, thr, rowinfo, nuc, total;
};

static SlLayout sl_layout(int B, int D, int V) {
  const size_t S = ((size_t)V + sd::kSlChunk - 1) / sd::kSlChunk, R = 2 * (size_t)D + 1;
  const size_t Ss = ((size_t)V + sd::kSlStatChunk - 1) / sd::kSlStatChunk;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  SlLayout l;
  l.stats = 0;
  l.gath = up((size_t)B * R * Ss * 16);
  l.part = l.gath + up((size_t)B * D * 8);
  l.thr = l.part + up((size_t)B * S * 16);
  l.rowinfo = l.thr + up((size_t)B * S * sd::kSlThreads * 16);
  l.nuc = l.rowinfo + up((size_t)B * 64);
  l.total = l.nuc + up((size_t)B * R * 32);
  return l;
}

EXPORT size_t specdec_sample_workspace_bytes(int B, int D, int V) {
  if (B < 0 || D < 0 || V < 1) return 0;
  return sl_layout(B, D, V).total;
}

EXPORT int specdec_verify_sample_logits(const void *target, const void *draft_logits, int dtype, int B, int D,
                                        int V, float temperature, float top_p, const int32_t *draft,
                                        const float *u_accept, const float *u_draw, int32_t *accept_len,
                                        int32_t *next_token, float *cutoff, void *ws, size_t ws_bytes,
                                        int32_t *status, void *stream) {
  if (B < 0 || B > 65535 || D < 0 || D > 255 || V < 1 || V > (1 << 22)) return SPECDEC_E_ARG;
  if (!(temperature > 0.0f) || !isfinite(temperature) || !(top_p > 0.0f) || top_p > 1.0f) return SPECDEC_E_ARG;
  if (dtype != SPECDEC_F32 && dtype != SPECDEC_F16 && dtype != SPECDEC_BF16) return SPECDEC_E_DTYPE;
  if (B == 0) return SPECDEC_OK;
  if (!target || !u_draw || !accept_len || !next_token || (D > 0 && (!draft_logits || !draft || !u_accept)))
    return SPECDEC_E_ARG;
  const SlLayout l = sl_layout(B, D, V);
  if (!ws || ws_bytes < l.total) return SPECDEC_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return SPECDEC_E_ALIGN;
  sd::SampleLogitsParams s;
  s.target = target;
  s.draftl = draft_logits;
  s.dtype = dtype;
  s.B = B;
  s.D = D;
  s.V = V;
  s.S = (int)((V + sd::kSlChunk - 1) / sd::kSlChunk);
  s.Ss = (int)((V + sd::kSlStatChunk - 1) / sd::kSlStatChunk);
  s.inv_t = 1.0 / (double)temperature;
  s.top_p = top_p;
  s.nucleus = top_p < 1.0f;
  s.cutoff = cutoff;
  s.draft = draft;
  s.u_accept = u_accept;
  s.u_draw = u_draw;
  s.accept_len = accept_len;
  s.next_token = next_token;
  s.status = status;
  char *w = static_cast<char *>(ws);
  s.stats = reinterpret_cast<double *>(w + l.stats);
  s.gath = reinterpret_cast<float *>(w + l.gath);
  s.part = reinterpret_cast<double *>(w + l.part);
  s.thr = reinterpret_cast<double *>(w + l.thr);
  s.rowinfo = reinterpret_cast<double *>(w + l.rowinfo);
  s.nuc = reinterpret_cast<double *>(w + l.nuc);
  const size_t e = dtype == SPECDEC_F32 ? 4 : 8;  // logits per 16-byte vector
  s.vec = (size_t)V % e == 0 && reinterpret_cast<uintptr_t>(target) % 16 == 0 &&
          (D == 0 || reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0);
  return launched(sd::launch_verify_sample_logits(s, as_stream(stream)));
}

// Host validation of a realignment call and its launch parameters.  Returns an
// error code, SPECDEC_OK with `p` filled, or kNothing when B = 0.
constexpr int kNothing = 1;

static int realign_prepare(int mode, const specdec_seqbuf_t *in, const specdec_seqbuf_t *out, const int32_t *rows,
                           int B, int group, const int32_t *skip_group, int D, const void *kv_new,
                           const int32_t *draft, const int32_t *accept_len, const int32_t *next_token,
                           int32_t pad_token, int32_t *status, sd::RealignParams &p) {
  if (mode != SPECDEC_EQSPEC && mode != SPECDEC_GATHER && mode != SPECDEC_APPEND_INPLACE &&
      mode != SPECDEC_EQSPEC_INPLACE && mode != SPECDEC_EQSPEC_INPLACE_ZERO_PAD)
    return SPECDEC_E_ARG;
  if (B < 0 || B > sd::kMaxRealignRows || D < 0) return SPECDEC_E_ARG;
  int rc = check_seqbuf_shape(in);
  if (rc) return rc;
  rc = check_seqbuf_shape(out);
  if (rc) return rc;
  if (!same_geometry(in, out)) return SPECDEC_E_ARG;
  const int units = (int)((size_t)in->head_dim * esize(in->dtype) / 16);
  if (units > 256) return SPECDEC_E_ARG;
  // one (layer, K|V, row, head) sequence is addressed with 32-bit byte offsets
  if ((size_t)in->cap * units * 16 >= (1u << 31) || (size_t)out->cap * units * 16 >= (1u << 31) ||
      ((size_t)D + 1) * units * 16 >= (1u << 31))
    return SPECDEC_E_ARG;
  // tiles are numbered with 32-bit integers
  if ((size_t)out->layers * 2 * (size_t)(out->rows > B ? out->rows : B) * out->heads * ((size_t)out->cap + 1) >=
      (1u << 31))
    return SPECDEC_E_ARG;

  memset(&p, 0, sizeof(p));
  p.mode = mode;
  p.kv_in = in->kv;
  p.kv_out = out->kv;
  p.kv_new = kv_new;
  p.layers = in->layers;
  p.heads = in->heads;
  p.units = units;
  p.rows_in = in->rows;
  p.cap_in = in->cap;
  p.rows_out = out->rows;
  p.cap_out = out->cap;
  p.B = B;
  p.group = group;
  p.D = D;
  p.draft = draft;
  p.accept_len = accept_len;
  p.next_token = next_token;
  p.pad_token = pad_token;
  p.status = status;
  p.rows = rows;
  p.skip_group = skip_group;

  const size_t tok_in_bytes = (size_t)in->rows * in->cap * 4, tok_out_bytes = (size_t)out->rows * out->cap * 4;
  if (mode == SPECDEC_EQSPEC) {
    if (in->rows != B || out->rows != B) return SPECDEC_E_ARG;
    if (B == 0) return kNothing;
    if (!in->tokens || !in->width || !out->tokens || !out->pos || !out->mask || !out->width) return SPECDEC_E_ARG;
    if (!kv_new || !accept_len || !next_token || (D > 0 && !draft)) return SPECDEC_E_ARG;
    if (reinterpret_cast<uintptr_t>(kv_new) % 16 != 0) return SPECDEC_E_ALIGN;
    const size_t kin = kv_bytes(in), kout = kv_bytes(out);
    const size_t knew = (size_t)in->layers * 2 * B * in->heads * ((size_t)D + 1) * in->head_dim * esize(in->dtype);
    if (overlap(in->kv, kin, out->kv, kout) || overlap(kv_new, knew, out->kv, kout)) return SPECDEC_E_ALIAS;
    if (overlap(in->tokens, tok_in_bytes, out->tokens, tok_out_bytes) || overlap(in->len, B * 4u, out->len, B * 4u) ||
        overlap(in->width, 4, out->width, 4) || overlap(accept_len, B * 4u, out->len, B * 4u))
      return SPECDEC_E_ALIAS;
    p.tok_in = in->tokens;
    p.len_in = in->len;
    p.width_in = in->width;
    p.tok_out = out->tokens;
    p.pos_out = out->pos;
    p.mask_out = out->mask;
    p.len_out = out->len;
    p.width_out = out->width;
  } else if (mode == SPECDEC_EQSPEC_INPLACE || mode == SPECDEC_EQSPEC_INPLACE_ZERO_PAD) {
    if (in->rows != B || !same_buffers(in, out)) return SPECDEC_E_ARG;
    if (B == 0) return kNothing;
    if (!in->tokens || !in->pos || !in->mask || !in->width) return SPECDEC_E_ARG;
    if (!kv_new || !accept_len || !next_token || (D > 0 && !draft)) return SPECDEC_E_ARG;
    if (reinterpret_cast<uintptr_t>(kv_new) % 16 != 0) return SPECDEC_E_ALIGN;
    const size_t knew = (size_t)in->layers * 2 * B * in->heads * ((size_t)D + 1) * in->head_dim * esize(in->dtype);
    if (overlap(kv_new, knew, in->kv, kv_bytes(in))) return SPECDEC_E_ALIAS;
    if (overlap(accept_len, B * 4u, in->len, B * 4u) || overlap(next_token, B * 4u, in->tokens, tok_in_bytes) ||
        (D > 0 && overlap(draft, (size_t)B * D * 4, in->tokens, tok_in_bytes)))
      return SPECDEC_E_ALIAS;
    p.tok_in = in->tokens;
    p.len_in = in->len;
    p.width_in = in->width;
    p.tok_out = out->tokens;
    p.pos_out = out->pos;
    p.mask_out = out->mask;
    p.len_out = out->len;
    p.width_out = out->width;
  } else if (mode == SPECDEC_GATHER) {
    if (group < 1) return SPECDEC_E_ARG;
    if (out->rows < B) return SPECDEC_E_ARG;
    if (B == 0) return kNothing;
    if (overlap(in->kv, kv_bytes(in), out->kv, kv_bytes(out))) return SPECDEC_E_ALIAS;
    if (overlap(in->tokens, tok_in_bytes, out->tokens, tok_out_bytes)) return SPECDEC_E_ALIAS;
    p.tok_in = in->tokens;
    p.len_in = in->len;
    p.tok_out = out->tokens;
    p.pos_out = out->pos;
    p.mask_out = out->mask;
    p.len_out = out->len;
    p.width_out = out->width;
  } else {
    if (in->kv != out->kv || in->len != out->len || in->tokens != out->tokens || in->rows != out->rows ||
        in->cap != out->cap)
      return SPECDEC_E_ARG;
    if (B == 0) return kNothing;
    if (!kv_new || !accept_len || !next_token || (D > 0 && !draft)) return SPECDEC_E_ARG;
    if (reinterpret_cast<uintptr_t>(kv_new) % 16 != 0) return SPECDEC_E_ALIGN;
    const size_t knew = (size_t)in->layers * 2 * B * in->heads * ((size_t)D + 1) * in->head_dim * esize(in->dtype);
    if (overlap(kv_new, knew, in->kv, kv_bytes(in))) return SPECDEC_E_ALIAS;
    p.tok_in = in->tokens;
    p.len_in = in->len;
    p.tok_out = out->tokens;
    p.len_out = out->len;
  }
  return SPECDEC_OK;
}

EXPORT int specdec_realign_kv(int mode, const specdec_seqbuf_t *in, const specdec_seqbuf_t *out,
                              const int32_t *rows, int B, int group, const int32_t *skip_group, int D,
                              const void *kv_new, const int32_t *draft, const int32_t *accept_len,
                              const int32_t *next_token, int32_t pad_token, int32_t *status, void *stream) {
  sd::RealignParams p;
  const int rc = realign_prepare(mode, in, out, rows, B, group, skip_group, D, kv_new, draft, accept_len, next_token,
                                 pad_token, status, p);
  if (rc != SPECDEC_OK) return rc == kNothing ? SPECDEC_OK : rc;
  const bool inplace = mode == SPECDEC_EQSPEC_INPLACE || mode == SPECDEC_EQSPEC_INPLACE_ZERO_PAD;
  return launched(inplace ? sd::launch_realign_inplace(p, as_stream(stream)) : sd::launch_realign(p, as_stream(stream)));
}

EXPORT int specdec_group_by_len(const int32_t *len, int N, int group, int32_t *order, int32_t *uniform,
                                int32_t *width, int32_t *n_uniform, void *stream) {
  if (N < 0 || N > kMaxPool || group < 1) return SPECDEC_E_ARG;
  if (!n_uniform) return SPECDEC_E_ARG;
  if (N > 0 && (!len || !order || !uniform || !width)) return SPECDEC_E_ARG;
  sd::GroupParams p;
  p.len = len;
  p.ids = nullptr;
  p.N = N;
  p.group = group;
  p.order = order;
  p.uniform = uniform;
  p.width = width;
  p.n_uniform = n_uniform;
  return launched(sd::launch_group_by_len(p, as_stream(stream)));
}

// ------------------------------------------------------------------ paged KV

static_assert(SPECDEC_PAGED_SYNC_WORDS == sd::kPagedSyncWords, "the header states the counter words");

static int check_paged(const specdec_paged_t *k) {
  if (!k || !k->pages || !k->block_table || !k->free_pages || !k->n_free || !k->tokens || !k->len || !k->sync)
    return SPECDEC_E_ARG;
  if (k->rows < 1 || k->n_pages < 1 || k->page < 1 || k->max_blocks < 1 || k->layers < 0 || k->heads < 1 ||
      k->head_dim < 1)
    return SPECDEC_E_ARG;
  if (!dtype_ok(k->dtype)) return SPECDEC_E_DTYPE;
  if (((size_t)k->head_dim * esize(k->dtype)) % 16 != 0) return SPECDEC_E_ALIGN;
  if (reinterpret_cast<uintptr_t>(k->pages) % 16 != 0) return SPECDEC_E_ALIGN;
  // positions of a row and token offsets are 32-bit integers
  if ((size_t)k->max_blocks * (size_t)k->page >= (1u << 30)) return SPECDEC_E_ARG;
  return SPECDEC_OK;
}

static size_t paged_bytes(const specdec_paged_t *k) {
  return (size_t)k->layers * 2 * (size_t)k->n_pages * k->heads * (size_t)k->page * k->head_dim * esize(k->dtype);
}

static sd::PagedParams paged_params(int op, const specdec_paged_t *k, const int32_t *rows, int B, int32_t *status) {
  sd::PagedParams p;
  memset(&p, 0, sizeof(p));
  p.op = op;
  p.pages = k->pages;
  p.bt = k->block_table;
  p.free_pages = k->free_pages;
  p.n_free = k->n_free;
  p.tokens = k->tokens;
  p.len = k->len;
  p.sync = k->sync;
  p.layers = k->layers;
  p.heads = k->heads;
  p.units = (int)((size_t)k->head_dim * esize(k->dtype) / 16);
  p.n_pages = k->n_pages;
  p.page = k->page;
  p.max_blocks = k->max_blocks;
  p.rows = k->rows;
  p.rowmap = rows;
  p.B = B;
  p.status = status;
  return p;
}

static bool paged_matches(const specdec_paged_t *k, const specdec_seqbuf_t *s) {
  return s->layers == k->layers && s->heads == k->heads && s->head_dim == k->head_dim && s->dtype == k->dtype;
}

static int paged_append_prepare(const specdec_paged_t *kv, const int32_t *rows, int B, int D, const void *kv_new,
                                const int32_t *draft, const int32_t *accept_len, const int32_t *next_token,
                                int32_t pad_token, int32_t *width, int32_t *rect_tokens, int32_t *rect_pos,
                                int8_t *rect_mask, int rect_cap, int32_t *status, sd::PagedParams &p) {
  int rc = check_paged(kv);
  if (rc) return rc;
  if (B < 0 || B > sd::kMaxRealignRows || D < 0 || D > 255) return SPECDEC_E_ARG;
  if (B == 0) return kNothing;
  if (!kv_new || !accept_len || !next_token || (D > 0 && !draft)) return SPECDEC_E_ARG;
  if ((rect_tokens || rect_pos || rect_mask) && (!rect_tokens || rect_cap < 1)) return SPECDEC_E_ARG;
  if (reinterpret_cast<uintptr_t>(kv_new) % 16 != 0) return SPECDEC_E_ALIGN;
  const size_t knew = (size_t)kv->layers * 2 * B * kv->heads * ((size_t)D + 1) * kv->head_dim * esize(kv->dtype);
  if (knew / 16 >= (1u << 31)) return SPECDEC_E_ARG;  // kv_new units are numbered with 32-bit integers
  if (overlap(kv_new, knew, kv->pages, paged_bytes(kv))) return SPECDEC_E_ALIAS;
  p = paged_params(sd::kPagedAppend, kv, rows, B, status);
  p.D = D;
  p.kv_new = kv_new;
  p.draft = draft;
  p.accept_len = accept_len;
  p.next_token = next_token;
  p.pad_token = pad_token;
  p.width_out = width;
  p.rect_tok = rect_tokens;
  p.rect_pos = rect_pos;
  p.rect_mask = rect_mask;
  p.rect_cap = rect_cap;
  return SPECDEC_OK;
}

EXPORT int specdec_paged_append(const specdec_paged_t *kv, const int32_t *rows, int B, int D, const void *kv_new,
                                const int32_t *draft, const int32_t *accept_len, const int32_t *next_token,
                                int32_t pad_token, int32_t *width, int32_t *rect_tokens, int32_t *rect_pos,
                                int8_t *rect_mask, int rect_cap, int32_t *status, void *stream) {
  sd::PagedParams p;
  const int rc = paged_append_prepare(kv, rows, B, D, kv_new, draft, accept_len, next_token, pad_token, width,
                                      rect_tokens, rect_pos, rect_mask, rect_cap, status, p);
  if (rc != SPECDEC_OK) return rc == kNothing ? SPECDEC_OK : rc;
  return launched(sd::launch_paged(p, as_stream(stream)));
}

EXPORT int specdec_paged_gather(const specdec_paged_t *kv, const int32_t *rows, int B, const specdec_seqbuf_t *out,
                                int32_t pad_token, int32_t *status, void *stream) {
  int rc = check_paged(kv);
  if (rc) return rc;
  rc = check_seqbuf_shape(out);
  if (rc) return rc;
  if (B < 0 || B > sd::kMaxRealignRows || out->rows != B || !paged_matches(kv, out)) return SPECDEC_E_ARG;
  if (B == 0) return SPECDEC_OK;
  if (!out->tokens || !out->width || out->cap < 1) return SPECDEC_E_ARG;
  if (overlap(out->kv, kv_bytes(out), kv->pages, paged_bytes(kv))) return SPECDEC_E_ALIAS;
  sd::PagedParams p = paged_params(sd::kPagedGather, kv, rows, B, status);
  p.pad_token = pad_token;
  p.rect_kv = out->kv;
  p.rect_tok = out->tokens;
  p.rect_pos = out->pos;
  p.rect_mask = out->mask;
  p.rect_len = out->len;
  p.rect_width = out->width;
  p.rect_cap = out->cap;
  return launched(sd::launch_paged(p, as_stream(stream)));
}

EXPORT int specdec_paged_admit(const specdec_paged_t *kv, const int32_t *rows, int B, const specdec_seqbuf_t *in,
                               int32_t *status, void *stream) {
  int rc = check_paged(kv);
  if (rc) return rc;
  rc = check_seqbuf_shape(in);
  if (rc) return rc;
  if (B < 0 || B > sd::kMaxRealignRows || in->rows != B || !paged_matches(kv, in)) return SPECDEC_E_ARG;
  if (B == 0) return SPECDEC_OK;
  if (!in->tokens || !in->width) return SPECDEC_E_ARG;
  if (overlap(in->kv, kv_bytes(in), kv->pages, paged_bytes(kv))) return SPECDEC_E_ALIAS;
  sd::PagedParams p = paged_params(sd::kPagedAdmit, kv, rows, B, status);
  p.rect_kv = in->kv;
  p.rect_tok = in->tokens;
  p.rect_cap = in->cap;
  p.in_len = in->len;
  p.in_width = in->width;
  return launched(sd::launch_paged(p, as_stream(stream)));
}

EXPORT int specdec_paged_retire(const specdec_paged_t *kv, const int32_t *rows, int B, int32_t *status,
                                void *stream) {
  int rc = check_paged(kv);
  if (rc) return rc;
  if (B < 0 || B > sd::kMaxRealignRows) return SPECDEC_E_ARG;
  if (B == 0) return SPECDEC_OK;
  sd::PagedParams p = paged_params(sd::kPagedRetire, kv, rows, B, status);
  return launched(sd::launch_paged(p, as_stream(stream)));
}

// ------------------------------------------------------------ pool lifecycle

EXPORT int specdec_group_by_len_ids(const int32_t *len, const int32_t *ids, int N, int group, int32_t *order,
                                    int32_t *uniform, int32_t *width, int32_t *n_uniform, void *stream) {
  if (N < 0 || N > kMaxPool || group < 1) return SPECDEC_E_ARG;
  if (!n_uniform) return SPECDEC_E_ARG;
  if (N > 0 && (!len || !ids || !order || !uniform || !width)) return SPECDEC_E_ARG;
  sd::GroupParams p;
  p.len = len;
  p.ids = ids;
  p.N = N;
  p.group = group;
  p.order = order;
  p.uniform = uniform;
  p.width = width;
  p.n_uniform = n_uniform;
  return launched(sd::launch_group_by_len(p, as_stream(stream)));
}

static bool sched_ok(const specdec_sched_t *s) {
  return s && s->active && s->n_active && s->free_slots && s->n_free && s->q_head;
}

static sd::PoolParams pool_params(const specdec_seqbuf_t *pool, const specdec_sched_t *st, int32_t *status) {
  sd::PoolParams p;
  memset(&p, 0, sizeof(p));
  p.kv = pool->kv;
  p.tokens = pool->tokens;
  p.len = pool->len;
  p.layers = pool->layers;
  p.heads = pool->heads;
  p.units = (int)((size_t)pool->head_dim * esize(pool->dtype) / 16);
  p.slots = pool->rows;
  p.cap = pool->cap;
  p.active = st->active;
  p.n_active = st->n_active;
  p.free_slots = st->free_slots;
  p.n_free = st->n_free;
  p.q_head = st->q_head;
  p.status = status;
  return p;
}

EXPORT int specdec_pool_finish(const specdec_seqbuf_t *pool, const specdec_sched_t *sched, const int32_t *rows,
                               const int32_t *accept_len, int B, int D, int32_t eos_id, int32_t max_len,
                               int32_t *retired, int32_t *n_retired, int32_t *status, void *stream) {
  int rc = check_seqbuf_shape(pool);
  if (rc) return rc;
  if (!sched_ok(sched) || !pool->tokens || !retired || !n_retired) return SPECDEC_E_ARG;
  if (pool->rows < 1 || pool->rows > sd::kMaxPoolSlots || B < 0 || B > pool->rows || D < 0 || max_len < 1)
    return SPECDEC_E_ARG;
  if (B > 0 && (!rows || !accept_len)) return SPECDEC_E_ARG;
  sd::PoolParams p = pool_params(pool, sched, status);
  p.rows = rows;
  p.accept_len = accept_len;
  p.B = B;
  p.D = D;
  p.eos_id = eos_id;
  p.max_len = max_len;
  p.retired = retired;
  p.n_retired = n_retired;
  return launched(sd::launch_pool_finish(p, as_stream(stream)));
}

EXPORT int specdec_pool_admit(const specdec_seqbuf_t *pool, const specdec_sched_t *sched, const specdec_seqbuf_t *queue,
                              int32_t *admitted, int32_t *n_admitted, int32_t *status, void *stream) {
  int rc = check_seqbuf_shape(pool);
  if (rc) return rc;
  rc = check_seqbuf_shape(queue);
  if (rc) return rc;
  if (!sched_ok(sched) || !pool->tokens || (!queue->tokens && queue->rows > 0) || !admitted || !n_admitted)
    return SPECDEC_E_ARG;
  if (pool->rows < 1 || pool->rows > sd::kMaxPoolSlots || queue->cap < 1 || !same_geometry(pool, queue))
    return SPECDEC_E_ARG;
  if (overlap(queue->kv, kv_bytes(queue), pool->kv, kv_bytes(pool))) return SPECDEC_E_ALIAS;
  sd::PoolParams p = pool_params(pool, sched, status);
  p.pkv = queue->kv;
  p.ptok = queue->tokens;
  p.plen = queue->len;
  p.Q = queue->rows;
  p.pcap = queue->cap;
  p.admitted = admitted;
  p.n_admitted = n_admitted;
  return launched(sd::launch_pool_admit(p, as_stream(stream)));
}
