"""Python binding of libspecdec (include/specdec.h).

Argument marshalling only: tensors are checked for device, dtype and layout,
their device pointers and torch's current HIP stream are handed to the C ABI,
and every step runs in the library's HIP kernels.  There is no fallback: if the
library is missing, calls raise.
"""
import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecdec.so")

F32, F16, BF16 = 0, 1, 2
EQSPEC, GATHER, APPEND_INPLACE, EQSPEC_INPLACE, EQSPEC_INPLACE_ZERO_PAD = 0, 1, 2, 3, 4
OK, E_ARG, E_DTYPE, E_WORKSPACE, E_ALIAS, E_ALIGN, E_LAUNCH, E_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
S_DRAFT_RANGE, S_CAPACITY, S_LEN_RANGE, S_PROB, S_ROWS_DUP = 1, 2, 4, 8, 16

_ERRORS = {E_ARG: "invalid argument", E_DTYPE: "unsupported element type", E_WORKSPACE: "workspace too small",
           E_ALIAS: "output overlaps an input", E_ALIGN: "misaligned KV buffer", E_LAUNCH: "kernel launch failed",
           E_SCRATCH: "batch too large for the library's static scratch"}
_TORCH_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

EXPORTS = ("specdec_version", "specdec_workspace_bytes", "specdec_workspace_init", "specdec_verify_greedy",
           "specdec_verify_sample", "specdec_sample_workspace_bytes", "specdec_verify_sample_logits",
           "specdec_realign_kv", "specdec_group_by_len", "specdec_paged_append", "specdec_paged_gather",
           "specdec_paged_admit", "specdec_paged_retire", "specdec_group_by_len_ids", "specdec_pool_finish",
           "specdec_pool_admit", "specdec_verify_greedy_noalloc", "specdec_verify_sample_workspace_bytes")


class SpecDecError(RuntimeError):
    def __init__(self, code, where):
        super().__init__("%s: %s (code %d)" % (where, _ERRORS.get(code, "error"), code))
        self.code = code


class SeqBufC(C.Structure):
    _fields_ = [("kv", C.c_void_p), ("tokens", C.c_void_p), ("pos", C.c_void_p), ("mask", C.c_void_p),
                ("len", C.c_void_p), ("width", C.c_void_p), ("rows", C.c_int32), ("cap", C.c_int32),
                ("layers", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int32)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libspecdec.so is not built (run __graft_entry__.build()); there is no fallback")
        L = C.CDLL(LIB_PATH)
        vp, ci, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
        L.specdec_version.restype = C.c_char_p
        L.specdec_workspace_bytes.argtypes = [ci, ci]
        L.specdec_workspace_bytes.restype = sz
        L.specdec_workspace_init.argtypes = [vp, sz, vp]
        L.specdec_verify_greedy.argtypes = [vp, ci, i64, ci, ci, ci, vp, vp, vp, vp, vp, sz, vp, vp]
        L.specdec_verify_greedy_noalloc.argtypes = [vp, ci, i64, ci, ci, ci, vp, vp, vp, vp, vp, vp]
        L.specdec_verify_sample.argtypes = [vp, vp, ci, ci, ci, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.specdec_verify_sample_workspace_bytes.argtypes = [ci, ci, ci]
        L.specdec_verify_sample_workspace_bytes.restype = sz
        L.specdec_sample_workspace_bytes.argtypes = [ci, ci, ci]
        L.specdec_sample_workspace_bytes.restype = sz
        L.specdec_verify_sample_logits.argtypes = [vp, vp, ci, ci, ci, ci, C.c_float, C.c_float, vp, vp, vp, vp, vp,
                                                   vp, vp, sz, vp, vp]
        L.specdec_realign_kv.argtypes = [ci, C.POINTER(SeqBufC), C.POINTER(SeqBufC), vp, ci, ci, vp, ci, vp, vp,
                                         vp, vp, C.c_int32, vp, vp]
        L.specdec_group_by_len.argtypes = [vp, ci, ci, vp, vp, vp, vp, vp]
        L.specdec_paged_append.argtypes = [C.POINTER(PagedC), vp, ci, ci, vp, vp, vp, vp, C.c_int32, vp, vp, vp,
                                           vp, ci, vp, vp]
        L.specdec_paged_gather.argtypes = [C.POINTER(PagedC), vp, ci, C.POINTER(SeqBufC), C.c_int32, vp, vp]
        L.specdec_paged_admit.argtypes = [C.POINTER(PagedC), vp, ci, C.POINTER(SeqBufC), vp, vp]
        L.specdec_paged_retire.argtypes = [C.POINTER(PagedC), vp, ci, vp, vp]
        L.specdec_group_by_len_ids.argtypes = [vp, vp, ci, ci, vp, vp, vp, vp, vp]
        L.specdec_pool_finish.argtypes = [C.POINTER(SeqBufC), C.POINTER(SchedC), vp, vp, ci, ci, C.c_int32, C.c_int32,
                                          vp, vp, vp, vp]
        L.specdec_pool_admit.argtypes = [C.POINTER(SeqBufC), C.POINTER(SchedC), C.POINTER(SeqBufC), vp, vp, vp, vp]
        for f in ("specdec_workspace_init", "specdec_verify_greedy", "specdec_verify_greedy_noalloc",
                  "specdec_verify_sample",
                  "specdec_verify_sample_logits", "specdec_realign_kv", "specdec_group_by_len",
                  "specdec_paged_append", "specdec_paged_gather", "specdec_paged_admit", "specdec_paged_retire",
                  "specdec_group_by_len_ids", "specdec_pool_finish", "specdec_pool_admit"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, cuda=True):
    if t is None:
        raise ValueError("%s is required" % name)
    if cuda and not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _out(t, name, n, dtype=torch.int32, device=None):
    """A caller-supplied output (or None): a contiguous device tensor of `dtype`
    with room for n elements, on `device` when given."""
    if t is None:
        return None
    _need(t, name, dtype)
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s" % (name, device))
    if t.numel() < n:
        raise ValueError("%s needs at least %d elements, has %d" % (name, n, t.numel()))
    return t


def _check(rc, where):
    if rc != OK:
        raise SpecDecError(rc, where)


def specdec_version():
    return lib().specdec_version().decode()


def workspace(B, D, device="cuda"):
    """A cleared verification workspace for B rows and D drafts."""
    n = int(lib().specdec_workspace_bytes(B, D))
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    _check(lib().specdec_workspace_init(ws.data_ptr(), ws.numel(), _stream()), "specdec_workspace_init")
    return ws


def _i32(shape, device):
    return torch.empty(shape, dtype=torch.int32, device=device)


def _greedy_shape(logits, draft):
    """(B, D, V, row_stride) of a greedy verification, after the tensor checks."""
    if logits.dtype not in _TORCH_DT or not logits.is_cuda or logits.dim() != 3:
        raise ValueError("logits must be a [B, D+1, V] float32/float16/bfloat16 device tensor")
    B, D1, V = logits.shape
    D = D1 - 1
    if logits.stride(2) != 1:
        raise ValueError("logits must have a contiguous last dimension")
    if D1 == 1:
        row_stride = logits.stride(0)
    else:
        row_stride = logits.stride(1)
        if B > 1 and logits.stride(0) != D1 * row_stride:
            raise ValueError("logits rows must share one stride")
    _need(draft, "draft", torch.int32)
    if tuple(draft.shape) != (B, D):
        raise ValueError("draft must be [B, D]")
    return B, D, V, row_stride


def specdec_verify_greedy(logits, draft, ws=None, status=None, accept_len=None, next_token=None, target_tok=None):
    """Greedy verification of drafts [B, D] against logits [B, D+1, V].

    Rows of `logits` may be strided (last dim contiguous, a uniform stride
    between the B*(D+1) rows).  Returns (accept_len [B], next_token [B]).
    """
    B, D, V, row_stride = _greedy_shape(logits, draft)
    dev = logits.device
    ws = workspace(B, D, dev) if ws is None else _out(ws, "ws", 1, torch.uint8, device=dev)
    accept_len = _i32(B, dev) if accept_len is None else _out(accept_len, "accept_len", B, device=dev)
    next_token = _i32(B, dev) if next_token is None else _out(next_token, "next_token", B, device=dev)
    _out(target_tok, "target_tok", B * (D + 1), device=dev)
    _out(status, "status", 1, device=dev)
    rc = lib().specdec_verify_greedy(logits.data_ptr(), _TORCH_DT[logits.dtype], row_stride, B, D, V, _ptr(draft),
                                     _ptr(accept_len), _ptr(next_token), _ptr(target_tok), ws.data_ptr(),
                                     ws.numel(), _ptr(status), _stream())
    _check(rc, "specdec_verify_greedy")
    return accept_len, next_token


def specdec_verify_greedy_noalloc(logits, draft, accept_len, next_token, status=None, target_tok=None):
    """Greedy verification with the library's static workspace: the caller
    passes every output, and the call allocates nothing (no torch tensor
    either).  Returns (accept_len, next_token)."""
    B, D, V, row_stride = _greedy_shape(logits, draft)
    dev = logits.device
    _out(accept_len, "accept_len", B, device=dev)
    _out(next_token, "next_token", B, device=dev)
    if accept_len is None or next_token is None:
        raise ValueError("accept_len and next_token are required")
    _out(target_tok, "target_tok", B * (D + 1), device=dev)
    _out(status, "status", 1, device=dev)
    rc = lib().specdec_verify_greedy_noalloc(logits.data_ptr(), _TORCH_DT[logits.dtype], row_stride, B, D, V,
                                             _ptr(draft), _ptr(accept_len), _ptr(next_token), _ptr(target_tok),
                                             _ptr(status), _stream())
    _check(rc, "specdec_verify_greedy_noalloc")
    return accept_len, next_token


def sample_verify_workspace(B, D, V, device="cuda"):
    """A cleared workspace for sampled verification of B rows, D drafts, V ids
    (reusable by later calls on the same stream)."""
    n = int(lib().specdec_verify_sample_workspace_bytes(B, D, V))
    if n == 0:
        raise SpecDecError(E_ARG, "specdec_verify_sample_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check(lib().specdec_workspace_init(ws.data_ptr(), ws.numel(), _stream()), "specdec_workspace_init")
    return ws


def specdec_verify_sample(p, q, draft, u_accept, u_draw, status=None, accept_len=None, next_token=None, ws=None):
    """Sampled verification: p [B, D+1, V], q [B, D, V] float32 probabilities,
    uniforms u_accept [B, D] and u_draw [B, D+1].  Returns (accept_len, next_token)."""
    _need(p, "p", torch.float32)
    B, D1, V = p.shape
    D = D1 - 1
    _need(q, "q", torch.float32)
    _need(draft, "draft", torch.int32)
    _need(u_accept, "u_accept", torch.float32)
    _need(u_draw, "u_draw", torch.float32)
    if tuple(q.shape) != (B, D, V) or tuple(draft.shape) != (B, D) or tuple(u_accept.shape) != (B, D) or \
            tuple(u_draw.shape) != (B, D1):
        raise ValueError("shape mismatch between p, q, draft and the uniforms")
    dev = p.device
    accept_len = _i32(B, dev) if accept_len is None else _out(accept_len, "accept_len", B, device=dev)
    next_token = _i32(B, dev) if next_token is None else _out(next_token, "next_token", B, device=dev)
    _out(status, "status", 1, device=dev)
    if B == 0:
        ws_ptr, ws_n = None, 0
    else:
        ws = sample_verify_workspace(B, D, V, dev) if ws is None else _out(ws, "ws", 1, torch.uint8, device=dev)
        ws_ptr, ws_n = ws.data_ptr(), ws.numel()
    rc = lib().specdec_verify_sample(p.data_ptr(), q.data_ptr(), B, D, V, draft.data_ptr(), u_accept.data_ptr(),
                                     u_draw.data_ptr(), _ptr(accept_len), _ptr(next_token), ws_ptr, ws_n,
                                     _ptr(status), _stream())
    _check(rc, "specdec_verify_sample")
    return accept_len, next_token


def sample_workspace(B, D, V, device="cuda"):
    """Scratch workspace of sampled verification from logits (nothing kept between calls)."""
    n = int(lib().specdec_sample_workspace_bytes(B, D, V))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def specdec_verify_sample_logits(target, draft_logits, draft, u_accept, u_draw, temperature, top_p=1.0, ws=None,
                                 status=None, accept_len=None, next_token=None, cutoff=None):
    """Sampled verification from logits: target [B, D+1, V] and draft_logits [B, D, V]
    (float32, float16 or bfloat16), turned into p and q by the temperature and
    top-p on the device.  Returns (accept_len, next_token); `cutoff` (float32
    [B, 2D+1], optional) receives every row's nucleus threshold."""
    _need(target, "target")
    if target.dtype not in _TORCH_DT or target.dim() != 3:
        raise ValueError("target must be a [B, D+1, V] float32/float16/bfloat16 tensor")
    B, D1, V = target.shape
    D = D1 - 1
    _need(draft_logits, "draft_logits", target.dtype)
    _need(draft, "draft", torch.int32)
    _need(u_accept, "u_accept", torch.float32)
    _need(u_draw, "u_draw", torch.float32)
    if tuple(draft_logits.shape) != (B, D, V) or tuple(draft.shape) != (B, D) or \
            tuple(u_accept.shape) != (B, D) or tuple(u_draw.shape) != (B, D1):
        raise ValueError("shape mismatch between the logits, draft and the uniforms")
    dev = target.device
    ws = sample_workspace(B, D, V, dev) if ws is None else _out(ws, "ws", 1, torch.uint8, device=dev)
    accept_len = _i32(B, dev) if accept_len is None else _out(accept_len, "accept_len", B, device=dev)
    next_token = _i32(B, dev) if next_token is None else _out(next_token, "next_token", B, device=dev)
    _out(status, "status", 1, device=dev)
    if cutoff is not None:
        _need(cutoff, "cutoff", torch.float32)
        if cutoff.numel() != B * (2 * D + 1):
            raise ValueError("cutoff must hold B * (2D+1) floats")
    rc = lib().specdec_verify_sample_logits(target.data_ptr(), draft_logits.data_ptr(), _TORCH_DT[target.dtype], B,
                                            D, V, float(temperature), float(top_p), draft.data_ptr(),
                                            u_accept.data_ptr(), u_draw.data_ptr(), _ptr(accept_len),
                                            _ptr(next_token), _ptr(cutoff), ws.data_ptr(), ws.numel(), _ptr(status),
                                            _stream())
    _check(rc, "specdec_verify_sample_logits")
    return accept_len, next_token


class SeqBuf:
    """Device tensors of a sequence set: a left-padded rectangle or a pool.

    kv [L, 2, rows, H, cap, Dh]; tokens/pos [rows, cap] int32; mask [rows, cap]
    int8; len [rows] int32; width [groups] int32 (None for a pool)."""

    def __init__(self, kv, tokens, len, pos=None, mask=None, width=None):
        _need(kv, "kv")
        if kv.dtype not in _TORCH_DT or kv.dim() != 6 or kv.shape[1] != 2:
            raise ValueError("kv must be a [L, 2, rows, H, cap, Dh] float32/float16/bfloat16 tensor")
        self.kv, self.tokens, self.len, self.pos, self.mask, self.width = kv, tokens, len, pos, mask, width
        L, _, rows, H, cap, Dh = kv.shape
        for t, n, dt in ((tokens, "tokens", torch.int32), (pos, "pos", torch.int32), (mask, "mask", torch.int8)):
            if t is not None:
                _need(t, n, dt)
                if tuple(t.shape) != (rows, cap):
                    raise ValueError("%s must be [rows, cap]" % n)
        _need(len, "len", torch.int32)
        if len.numel() != rows:
            raise ValueError("len must hold one length per row")
        if width is not None:
            _need(width, "width", torch.int32)
            if width.numel() < 1:
                raise ValueError("width needs at least one entry")
        for t in (tokens, len, pos, mask, width):
            if t is not None and t.device != kv.device:
                raise ValueError("every tensor of a SeqBuf must be on the KV's device")
        self.c = SeqBufC(kv.data_ptr(), _ptr(tokens), _ptr(pos), _ptr(mask), len.data_ptr(), _ptr(width), rows, cap,
                         L, H, Dh, _TORCH_DT[kv.dtype])

    @property
    def rows(self):
        return self.kv.shape[2]

    @property
    def cap(self):
        return self.kv.shape[4]

    @staticmethod
    def empty(layers, rows, heads, cap, head_dim, dtype, device="cuda", groups=1, pool=False):
        kv = torch.empty((layers, 2, rows, heads, cap, head_dim), dtype=dtype, device=device)
        tok = torch.zeros((rows, cap), dtype=torch.int32, device=device)
        ln = torch.zeros(rows, dtype=torch.int32, device=device)
        if pool:
            return SeqBuf(kv, tok, ln)
        pos = torch.zeros((rows, cap), dtype=torch.int32, device=device)
        mask = torch.zeros((rows, cap), dtype=torch.int8, device=device)
        width = torch.zeros(max(groups, 1), dtype=torch.int32, device=device)
        return SeqBuf(kv, tok, ln, pos, mask, width)


def specdec_realign_kv(mode, src, dst, rows=None, B=None, group=0, skip_group=None, kv_new=None, draft=None,
                       accept_len=None, next_token=None, pad_token=0, status=None):
    """Realignment in one of the modes EQSPEC, GATHER, APPEND_INPLACE (see include/specdec.h)."""
    if B is None:
        B = rows.numel() if rows is not None else src.rows
    D = 0
    if kv_new is not None:
        _need(kv_new, "kv_new", src.kv.dtype)
        D = kv_new.shape[4] - 1
    elif draft is not None:
        D = draft.shape[1]
    for t, n in ((rows, "rows"), (skip_group, "skip_group"), (draft, "draft"), (accept_len, "accept_len"),
                 (next_token, "next_token"), (status, "status")):
        if t is not None:
            _need(t, n, torch.int32)
    L, _, _, H, _, Dh = src.kv.shape
    if kv_new is not None and tuple(kv_new.shape) != (L, 2, B, H, D + 1, Dh):
        raise ValueError("kv_new must be [L, 2, B, H, D+1, Dh]")
    for t, n, shape in ((draft, "draft", (B, D)), (accept_len, "accept_len", (B,)), (next_token, "next_token", (B,)),
                        (rows, "rows", (B,))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError("%s must have shape %s" % (n, shape))
    _out(status, "status", 1)
    if mode == GATHER:
        ng = (B + group - 1) // max(group, 1)
        if skip_group is not None and skip_group.numel() < ng:
            raise ValueError("skip_group needs one entry per group")
        if dst.width is not None and dst.width.numel() < ng:
            raise ValueError("the rectangle's width tensor needs one entry per group")
    if mode in (EQSPEC, EQSPEC_INPLACE, EQSPEC_INPLACE_ZERO_PAD) and (src.width is None or dst.width is None or dst.pos is None or
                                             dst.mask is None):
        raise ValueError("EQSPEC needs width on both sides and pos/mask on the output")
    rc = lib().specdec_realign_kv(mode, C.byref(src.c), C.byref(dst.c), _ptr(rows), B, group, _ptr(skip_group), D,
                                  _ptr(kv_new), _ptr(draft), _ptr(accept_len), _ptr(next_token), pad_token,
                                  _ptr(status), _stream())
    _check(rc, "specdec_realign_kv")


def realign_eqspec(src, dst, kv_new, draft, accept_len, next_token, pad_token=0, status=None):
    """EQSPEC unpad-append-repad of rectangle `src` into rectangle `dst`."""
    specdec_realign_kv(EQSPEC, src, dst, None, src.rows, 0, None, kv_new, draft, accept_len, next_token,
                       pad_token, status)


def realign_eqspec_inplace(buf, kv_new, draft, accept_len, next_token, pad_token=0, status=None, zero_pad=False):
    """EQSPEC unpad-append-repad of rectangle `buf` in place.  Its pad must hold
    zero KV bytes, unless zero_pad=True, which writes the whole new pad with
    zeros (for the first round after a prefill that wrote KV at pad positions)."""
    specdec_realign_kv(EQSPEC_INPLACE_ZERO_PAD if zero_pad else EQSPEC_INPLACE, buf, buf, None, buf.rows, 0, None,
                       kv_new, draft, accept_len, next_token, pad_token, status)


def gather(pool, rect, rows, group, skip_group=None, pad_token=0, status=None):
    """Left-padded rectangles of the listed pool rows, one per group of `group` entries."""
    specdec_realign_kv(GATHER, pool, rect, rows, rows.numel() if rows is not None else pool.rows, group,
                       skip_group, None, None, None, None, pad_token, status)


def append(pool, kv_new, draft, accept_len, next_token, rows=None, status=None):
    """In-place append of every entry's committed tokens and KV at its pool row's length."""
    B = kv_new.shape[2]
    specdec_realign_kv(APPEND_INPLACE, pool, pool, rows, B, 0, None, kv_new, draft, accept_len, next_token, 0,
                       status)


def specdec_group_by_len(lens, group, order=None, uniform=None, width=None, n_uniform=None, ids=None):
    """Equal-length grouping of a pool: returns (order, uniform, width, n_uniform) device tensors.
    With `ids` (pool rows), entry i is row ids[i], its length lens[ids[i]], and order lists rows."""
    _need(lens, "lens", torch.int32)
    N = lens.numel() if ids is None else ids.numel()
    nb = (N + group - 1) // group if group > 0 else 0
    dev = lens.device
    order = _i32(N, dev) if order is None else _out(order, "order", N, device=dev)
    uniform = _i32(max(nb, 1), dev) if uniform is None else _out(uniform, "uniform", nb, device=dev)
    width = _i32(max(nb, 1), dev) if width is None else _out(width, "width", nb, device=dev)
    n_uniform = _i32(1, dev) if n_uniform is None else _out(n_uniform, "n_uniform", 1, device=dev)
    if ids is None:
        rc = lib().specdec_group_by_len(lens.data_ptr(), N, group, order.data_ptr(), uniform.data_ptr(),
                                        width.data_ptr(), n_uniform.data_ptr(), _stream())
    else:
        _need(ids, "ids", torch.int32)
        rc = lib().specdec_group_by_len_ids(lens.data_ptr(), ids.data_ptr(), N, group, order.data_ptr(),
                                            uniform.data_ptr(), width.data_ptr(), n_uniform.data_ptr(), _stream())
    _check(rc, "specdec_group_by_len")
    return order, uniform[:nb], width[:nb], n_uniform


verify_greedy = specdec_verify_greedy
verify_greedy_noalloc = specdec_verify_greedy_noalloc
verify_sample = specdec_verify_sample
verify_sample_logits = specdec_verify_sample_logits
group_by_len = specdec_group_by_len


# ----------------------------------------------------------------- paged KV

PAGED_SYNC_WORDS = 4128  # SPECDEC_PAGED_SYNC_WORDS


class PagedC(C.Structure):
    _fields_ = [("pages", C.c_void_p), ("block_table", C.c_void_p), ("free_pages", C.c_void_p),
                ("n_free", C.c_void_p), ("tokens", C.c_void_p), ("len", C.c_void_p), ("sync", C.c_void_p),
                ("rows", C.c_int32),
                ("n_pages", C.c_int32), ("page", C.c_int32), ("max_blocks", C.c_int32), ("layers", C.c_int32),
                ("heads", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int32)]


class PagedKV:
    """Device tensors of a paged KV cache (see specdec_paged_t in include/specdec.h).

    pages [L, 2, n_pages, H, page, Dh]; block_table [rows, max_blocks] int32
    (-1 = none); free_pages [n_pages] int32 stack with n_free [1] entries in use;
    tokens [rows, max_blocks*page] int32; len [rows] int32; sync [PAGED_SYNC_WORDS]
    int32, zero (allocated here when not given)."""

    def __init__(self, pages, block_table, free_pages, n_free, tokens, len, sync=None):
        _need(pages, "pages")
        if pages.dtype not in _TORCH_DT or pages.dim() != 6 or pages.shape[1] != 2:
            raise ValueError("pages must be a [L, 2, n_pages, H, page, Dh] float32/float16/bfloat16 tensor")
        L, _, n_pages, H, page, Dh = pages.shape
        for t, n in ((block_table, "block_table"), (free_pages, "free_pages"), (n_free, "n_free"),
                     (tokens, "tokens"), (len, "len")):
            _need(t, n, torch.int32)
        rows, max_blocks = block_table.shape
        if tuple(free_pages.shape) != (n_pages,) or n_free.numel() != 1 or \
                tuple(tokens.shape) != (rows, max_blocks * page) or tuple(len.shape) != (rows,):
            raise ValueError("inconsistent paged-cache shapes")
        self.pages, self.block_table, self.free_pages, self.n_free = pages, block_table, free_pages, n_free
        self.tokens, self.len = tokens, len
        self.sync = torch.zeros(PAGED_SYNC_WORDS, dtype=torch.int32, device=pages.device) if sync is None else sync
        _need(self.sync, "sync", torch.int32)
        if self.sync.numel() < PAGED_SYNC_WORDS:
            raise ValueError("sync must hold %d int32 words" % PAGED_SYNC_WORDS)
        self.c = PagedC(pages.data_ptr(), block_table.data_ptr(), free_pages.data_ptr(), n_free.data_ptr(),
                        tokens.data_ptr(), len.data_ptr(), self.sync.data_ptr(), rows, n_pages, page, max_blocks,
                        L, H, Dh, _TORCH_DT[pages.dtype])

    @staticmethod
    def empty(layers, rows, heads, head_dim, n_pages, page, max_blocks, dtype, device="cuda", free_order=None):
        """An empty cache: every page free (stack order `free_order`, default 0..n_pages-1)."""
        pages = torch.zeros((layers, 2, n_pages, heads, page, head_dim), dtype=dtype, device=device)
        bt = torch.full((rows, max_blocks), -1, dtype=torch.int32, device=device)
        fp = (torch.arange(n_pages, dtype=torch.int32, device=device) if free_order is None
              else free_order.to(device=device, dtype=torch.int32).contiguous())
        nf = torch.full((1,), n_pages, dtype=torch.int32, device=device)
        tok = torch.zeros((rows, max_blocks * page), dtype=torch.int32, device=device)
        ln = torch.zeros(rows, dtype=torch.int32, device=device)
        return PagedKV(pages, bt, fp, nf, tok, ln)

    @property
    def page(self):
        return self.pages.shape[4]


def paged_append(cache, kv_new, draft, accept_len, next_token, rows=None, pad_token=0, width=None,
                 rect_tokens=None, rect_pos=None, rect_mask=None, status=None):
    """Realignment on a paged cache: append every entry's committed tokens and
    speculative KV at its length; optionally the [B, rect_cap] rectangle view."""
    _need(kv_new, "kv_new", cache.pages.dtype)
    L, _, B, H, D1, Dh = kv_new.shape
    D = D1 - 1
    if (L, H, Dh) != (cache.pages.shape[0], cache.pages.shape[3], cache.pages.shape[5]):
        raise ValueError("kv_new must be [L, 2, B, H, D+1, Dh] of the cache's geometry")
    for t, n, shape in ((draft, "draft", (B, D)), (accept_len, "accept_len", (B,)), (next_token, "next_token", (B,)),
                        (rows, "rows", (B,))):
        if t is not None:
            _need(t, n, torch.int32)
            if tuple(t.shape) != shape:
                raise ValueError("%s must have shape %s" % (n, shape))
    rect_cap = 0
    if rect_tokens is not None:
        _need(rect_tokens, "rect_tokens", torch.int32)
        rect_cap = rect_tokens.shape[1]
        for t, n, dt in ((rect_pos, "rect_pos", torch.int32), (rect_mask, "rect_mask", torch.int8)):
            if t is not None:
                _need(t, n, dt)
                if tuple(t.shape) != tuple(rect_tokens.shape):
                    raise ValueError("%s must match rect_tokens' shape" % n)
    _out(width, "width", 1)
    _out(status, "status", 1)
    rc = lib().specdec_paged_append(C.byref(cache.c), _ptr(rows), B, D, kv_new.data_ptr(), _ptr(draft),
                                    accept_len.data_ptr(), next_token.data_ptr(), pad_token, _ptr(width),
                                    _ptr(rect_tokens), _ptr(rect_pos), _ptr(rect_mask), rect_cap, _ptr(status),
                                    _stream())
    _check(rc, "specdec_paged_append")


def paged_gather(cache, out, rows=None, pad_token=0, status=None):
    """The batch's rows as the left-padded rectangle `out` (a SeqBuf with one row per entry)."""
    B = out.rows
    if rows is not None:
        _need(rows, "rows", torch.int32)
        if rows.numel() != B:
            raise ValueError("rows must name one pool row per rectangle row")
    _out(status, "status", 1)
    rc = lib().specdec_paged_gather(C.byref(cache.c), _ptr(rows), B, C.byref(out.c), pad_token, _ptr(status),
                                    _stream())
    _check(rc, "specdec_paged_gather")


def paged_admit(cache, rect, rows=None, status=None):
    """Empty pool rows receive the content of the left-padded rectangle `rect` (a SeqBuf)."""
    B = rect.rows
    if rows is not None:
        _need(rows, "rows", torch.int32)
        if rows.numel() != B:
            raise ValueError("rows must name one pool row per rectangle row")
    _out(status, "status", 1)
    rc = lib().specdec_paged_admit(C.byref(cache.c), _ptr(rows), B, C.byref(rect.c), _ptr(status), _stream())
    _check(rc, "specdec_paged_admit")


def paged_retire(cache, rows, status=None):
    """The listed rows return their pages to the free stack and become empty."""
    _need(rows, "rows", torch.int32)
    _out(status, "status", 1)
    rc = lib().specdec_paged_retire(C.byref(cache.c), rows.data_ptr(), rows.numel(), _ptr(status), _stream())
    _check(rc, "specdec_paged_retire")


# ------------------------------------------------------------ pool lifecycle

class SchedC(C.Structure):
    _fields_ = [("active", C.c_void_p), ("n_active", C.c_void_p), ("free_slots", C.c_void_p),
                ("n_free", C.c_void_p), ("q_head", C.c_void_p)]


class Sched:
    """Device scheduling state of a pool (see specdec_sched_t): active [slots] rows in
    schedule order (n_active valid), free_slots [slots] ascending (n_free valid), q_head."""

    def __init__(self, slots, active=(), device="cuda"):
        act = [int(a) for a in active]
        fr = [s for s in range(slots) if s not in set(act)]
        self.active = torch.zeros(slots, dtype=torch.int32, device=device)
        self.free_slots = torch.zeros(slots, dtype=torch.int32, device=device)
        if act:
            self.active[:len(act)] = torch.tensor(act, dtype=torch.int32)
        if fr:
            self.free_slots[:len(fr)] = torch.tensor(fr, dtype=torch.int32)
        self.n_active = torch.tensor([len(act)], dtype=torch.int32, device=device)
        self.n_free = torch.tensor([len(fr)], dtype=torch.int32, device=device)
        self.q_head = torch.zeros(1, dtype=torch.int32, device=device)
        self.c = SchedC(self.active.data_ptr(), self.n_active.data_ptr(), self.free_slots.data_ptr(),
                        self.n_free.data_ptr(), self.q_head.data_ptr())


def pool_finish(pool, sched, rows, accept_len, D, eos_id, max_len, retired=None, n_retired=None, status=None):
    """Finish sequences at end-of-sequence or max length after a round's append.
    Returns (retired, n_retired) device tensors."""
    _need(rows, "rows", torch.int32)
    _need(accept_len, "accept_len", torch.int32)
    B = rows.numel()
    if accept_len.numel() != B:
        raise ValueError("rows and accept_len must have one entry per batch entry")
    dev = pool.kv.device
    retired = _i32(pool.rows, dev) if retired is None else _out(retired, "retired", pool.rows, device=dev)
    n_retired = _i32(1, dev) if n_retired is None else _out(n_retired, "n_retired", 1, device=dev)
    _out(status, "status", 1, device=dev)
    rc = lib().specdec_pool_finish(C.byref(pool.c), C.byref(sched.c), rows.data_ptr(), accept_len.data_ptr(), B, D,
                                   eos_id, max_len, retired.data_ptr(), n_retired.data_ptr(), _ptr(status), _stream())
    _check(rc, "specdec_pool_finish")
    return retired, n_retired


def pool_admit(pool, sched, queue, admitted=None, n_admitted=None, status=None):
    """Admit queued prompts (a SeqBuf of left-aligned prompts) into the lowest free rows.
    Returns (admitted, n_admitted) device tensors."""
    dev = pool.kv.device
    admitted = _i32(pool.rows, dev) if admitted is None else _out(admitted, "admitted", pool.rows, device=dev)
    n_admitted = _i32(1, dev) if n_admitted is None else _out(n_admitted, "n_admitted", 1, device=dev)
    _out(status, "status", 1, device=dev)
    rc = lib().specdec_pool_admit(C.byref(pool.c), C.byref(sched.c), C.byref(queue.c), admitted.data_ptr(),
                                  n_admitted.data_ptr(), _ptr(status), _stream())
    _check(rc, "specdec_pool_admit")
    return admitted, n_admitted
