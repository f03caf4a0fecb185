"""Reference oracle for batch speculative decoding's verify-and-resynchronize
step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product library never calls it
and shares no code with it.  `liboracle.so` (oracle.c) holds the batched
reference; `brute.py` is a second, per-sequence numpy reference for tiny cases.

Every function is pinned by CPU tests against values the pages fix (their
worked examples), closed forms and brute force; see oracle.c for the passages
each one follows and the readings taken where the pages leave a choice.
"""
import contextlib
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
F32, F16, BF16 = 0, 1, 2
OK, E_ARG, E_CAPACITY, E_PRECOND = 0, -1, -2, -3

_libs = {}
_threaded = False


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__("oracle returned %d" % code)
        self.code = code


def use_threads(flag):
    """Route later calls to the OpenMP build (True) or the single-threaded one
    (False, the default).  Both compute the same bytes (a CPU test checks it);
    the threaded build times the oracle on all host cores and runs the
    every-layer checks of the full-size GPU tests, where one thread would take
    minutes."""
    global _threaded
    _threaded = bool(flag)


@contextlib.contextmanager
def threaded():
    """Calls inside the block use the OpenMP build."""
    prev = _threaded
    use_threads(True)
    try:
        yield
    finally:
        use_threads(prev)


def threads():
    """Threads the library in use may run its loops on."""
    return int(lib().oracle_threads())


def lib():
    name = "liboracle_omp.so" if _threaded else "liboracle.so"
    if name not in _libs:
        path = os.path.join(HERE, name)
        if not os.path.exists(path):
            from . import _build
            _build.build()
        L = C.CDLL(path)
        vp, i32p, i8p = C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int8)
        ci, i64 = C.c_int, C.c_int64
        L.oracle_verify_greedy.argtypes = [vp, ci, i64, ci, ci, ci, i32p, i32p, i32p, i32p]
        L.oracle_verify_sample.argtypes = [C.POINTER(C.c_float), C.POINTER(C.c_float), ci, ci, ci, i32p,
                                           C.POINTER(C.c_float), C.POINTER(C.c_float), i32p, i32p,
                                           C.POINTER(C.c_double)]
        L.oracle_verify_sample_logits.argtypes = [vp, vp, ci, ci, ci, ci, C.c_float, C.c_float,
                                                  C.POINTER(C.c_float), i32p, C.POINTER(C.c_float),
                                                  C.POINTER(C.c_float), i32p, i32p, C.POINTER(C.c_double),
                                                  C.POINTER(C.c_float)]
        L.oracle_softmax_row.argtypes = [vp, ci, ci, C.c_float, C.c_float, C.POINTER(C.c_float),
                                         C.POINTER(C.c_double)]
        L.oracle_realign_eqspec.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, vp, vp, vp, i32p, C.c_int32, i32p, i8p,
                                            i32p, i32p, i32p, C.c_int32, i32p, i32p, i8p, i32p, i32p]
        L.oracle_group_by_len.argtypes = [i32p, ci, ci, i32p, i32p, i32p, i32p]
        L.oracle_gather.argtypes = [ci, ci, ci, ci, ci, ci, vp, i32p, i32p, i32p, ci, ci, i32p, ci, vp, i32p, i32p,
                                    i8p, i32p, C.c_int32]
        L.oracle_append.argtypes = [ci, ci, ci, ci, ci, ci, vp, i32p, i32p, i32p, ci, ci, vp, i32p, i32p, i32p]
        for f in (L.oracle_verify_greedy, L.oracle_verify_sample, L.oracle_verify_sample_logits,
                  L.oracle_softmax_row, L.oracle_realign_eqspec, L.oracle_group_by_len, L.oracle_gather,
                  L.oracle_append):
            f.restype = C.c_int
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = C.c_int
        _libs[name] = L
    return _libs[name]


def _p(a, t=C.c_int32):
    return None if a is None else a.ctypes.data_as(C.POINTER(t))


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _check(rc):
    if rc != OK:
        raise OracleError(rc)


def _dtype_code(arr):
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.float16:
        return F16
    if arr.dtype == np.uint16 or arr.dtype == np.int16:
        return BF16  # raw bfloat16 bits
    raise TypeError("logits must be float32, float16 or raw bf16 bits (uint16)")


def verify_greedy(logits, draft, B, D, V, row_stride=None):
    """logits: [B*(D+1), row_stride] (float32 | float16 | uint16 bf16 bits)."""
    logits = np.ascontiguousarray(logits)
    row_stride = logits.shape[-1] if row_stride is None else row_stride
    draft = _i32(draft).reshape(-1)
    acc = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    tgt = np.empty(B * (D + 1), np.int32)
    _check(lib().oracle_verify_greedy(logits.ctypes.data, _dtype_code(logits), row_stride, B, D, V, _p(draft),
                                      _p(acc), _p(nxt), _p(tgt)))
    return acc, nxt, tgt.reshape(B, D + 1)


def verify_sample(p, q, draft, u_accept, u_draw):
    """p [B,D+1,V], q [B,D,V] float32; u_accept [B,D], u_draw [B,D+1] float32."""
    p = np.ascontiguousarray(p, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, D1, V = p.shape
    D = D1 - 1
    draft = _i32(draft).reshape(-1)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32).reshape(-1)
    ud = np.ascontiguousarray(u_draw, dtype=np.float32).reshape(-1)
    acc = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    mass = np.empty(B, np.float64)
    rc = lib().oracle_verify_sample(_p(p, C.c_float), _p(q, C.c_float), B, D, V, _p(draft), _p(ua, C.c_float),
                                    _p(ud, C.c_float), _p(acc), _p(nxt), _p(mass, C.c_double))
    if rc not in (OK, E_PRECOND):
        raise OracleError(rc)
    return acc, nxt, mass


def verify_sample_logits(target, draft_logits, draft, u_accept, u_draw, temperature, top_p=1.0, cut=None,
                         return_cut=False):
    """target [B,D+1,V] and draft_logits [B,D,V] logits (float32 | float16 | uint16 bf16 bits), turned into
    p and q with the same temperature and top-p; returns (accept_len, next_token, residual mass), and the
    nucleus thresholds applied [B, 2D+1] (target rows, then draft rows) with return_cut.  `cut` [B, 2D+1]
    forces those thresholds instead of computing them."""
    t = np.ascontiguousarray(target)
    d = np.ascontiguousarray(draft_logits)
    B, D1, V = t.shape
    D = D1 - 1
    if d.shape != (B, D, V) or d.dtype != t.dtype:
        raise ValueError("draft logits must be [B, D, V] of the target's dtype")
    draft = _i32(draft).reshape(-1)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32).reshape(-1)
    ud = np.ascontiguousarray(u_draw, dtype=np.float32).reshape(-1)
    if cut is not None:
        cut = np.ascontiguousarray(cut, dtype=np.float32).reshape(-1)
        if cut.size != B * (2 * D + 1):
            raise ValueError("cut must hold B * (2D+1) thresholds")
    acc = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    mass = np.empty(B, np.float64)
    used = np.empty((B, 2 * D + 1), np.float32)
    rc = lib().oracle_verify_sample_logits(t.ctypes.data, d.ctypes.data, _dtype_code(t), B, D, V,
                                           float(temperature), float(top_p), _p(cut, C.c_float), _p(draft),
                                           _p(ua, C.c_float), _p(ud, C.c_float), _p(acc), _p(nxt),
                                           _p(mass, C.c_double), _p(used, C.c_float))
    if rc not in (OK, E_PRECOND):
        raise OracleError(rc)
    return (acc, nxt, mass, used) if return_cut else (acc, nxt, mass)


def softmax_row(logits, temperature, top_p=1.0, cut=None):
    """The fp64 probabilities verify_sample_logits forms from one row of logits
    (with the nucleus threshold `cut` forced when given)."""
    a = np.ascontiguousarray(logits).reshape(-1)
    out = np.empty(a.shape[0], np.float64)
    c = None if cut is None else np.array([cut], np.float32)
    _check(lib().oracle_softmax_row(a.ctypes.data, _dtype_code(a), a.shape[0], float(temperature), float(top_p),
                                    _p(c, C.c_float), _p(out, C.c_double)))
    return out


def realign_eqspec(kv_in, kv_new, len_in, width_in, tok_in, mask_in, accept_len, next_token, draft,
                   cap_out=None, pad_token=0, kv_out=None, tok_out=None, pos_out=None, mask_out=None):
    """Unpad-append-repad of a left-padded rectangle.

    kv_in [L,2,B,H,cap_in,Dh]; kv_new [L,2,B,H,D+1,Dh]; tok_in/mask_in [B,cap_in].
    Output arrays are allocated (zero) unless passed in; only [0, width) of each
    row is written.  Returns dict(kv, tokens, pos, mask, len, width)."""
    L, two, B, H, cap_in, Dh = kv_in.shape
    D = kv_new.shape[4] - 1
    cap_out = cap_in if cap_out is None else cap_out
    es = kv_in.dtype.itemsize
    kv_in = np.ascontiguousarray(kv_in)
    kv_new = np.ascontiguousarray(kv_new, dtype=kv_in.dtype)
    if kv_out is None:
        kv_out = np.zeros((L, 2, B, H, cap_out, Dh), dtype=kv_in.dtype)
    tok_out = np.zeros((B, cap_out), np.int32) if tok_out is None else tok_out
    pos_out = np.zeros((B, cap_out), np.int32) if pos_out is None else pos_out
    mask_out = np.zeros((B, cap_out), np.int8) if mask_out is None else mask_out
    len_out = np.empty(B, np.int32)
    width_out = np.empty(1, np.int32)
    mask_in = None if mask_in is None else np.ascontiguousarray(mask_in, dtype=np.int8)
    tok_in = _i32(tok_in)
    rc = lib().oracle_realign_eqspec(L, H, Dh, es, B, cap_in, cap_out, D, kv_in.ctypes.data, kv_out.ctypes.data,
                                     kv_new.ctypes.data, _p(_i32(len_in)), int(width_in), _p(tok_in),
                                     _p(mask_in, C.c_int8), _p(_i32(accept_len)), _p(_i32(next_token)),
                                     _p(_i32(draft).reshape(-1)), pad_token, _p(tok_out), _p(pos_out),
                                     _p(mask_out, C.c_int8), _p(len_out), _p(width_out))
    _check(rc)
    return dict(kv=kv_out, tokens=tok_out, pos=pos_out, mask=mask_out, len=len_out, width=int(width_out[0]))


def group_by_len(lens, G):
    lens = _i32(lens)
    N = lens.shape[0]
    nb = (N + G - 1) // G
    order = np.empty(N, np.int32)
    uni = np.empty(max(nb, 1), np.int32)
    wid = np.empty(max(nb, 1), np.int32)
    nu = np.empty(1, np.int32)
    _check(lib().oracle_group_by_len(_p(lens), N, G, _p(order), _p(uni), _p(wid), _p(nu)))
    return order, uni[:nb], wid[:nb], int(nu[0])


def gather(kv_pool, tok_pool, len_pool, rows, G, skip_group, cap_out, pad_token=0, kv_out=None, tok_out=None,
           pos_out=None, mask_out=None, width_out=None):
    """Left-padded rectangles of the pool rows listed in `rows`, one per group of G."""
    L, two, N, H, cap_pool, Dh = kv_pool.shape
    rows = _i32(rows)
    B = rows.shape[0]
    ng = (B + G - 1) // G
    if kv_out is None:
        kv_out = np.zeros((L, 2, B, H, cap_out, Dh), dtype=kv_pool.dtype)
    tok_out = np.zeros((B, cap_out), np.int32) if tok_out is None else tok_out
    pos_out = np.zeros((B, cap_out), np.int32) if pos_out is None else pos_out
    mask_out = np.zeros((B, cap_out), np.int8) if mask_out is None else mask_out
    width_out = np.zeros(max(ng, 1), np.int32) if width_out is None else width_out
    _check(lib().oracle_gather(L, H, Dh, kv_pool.dtype.itemsize, N, cap_pool, np.ascontiguousarray(kv_pool).ctypes.data,
                               _p(_i32(tok_pool)), _p(_i32(len_pool)), _p(rows), B, G, _p(_i32(skip_group)), cap_out,
                               kv_out.ctypes.data, _p(tok_out), _p(pos_out), _p(mask_out, C.c_int8), _p(width_out),
                               pad_token))
    return dict(kv=kv_out, tokens=tok_out, pos=pos_out, mask=mask_out, width=width_out[:ng])


def append(kv_pool, tok_pool, len_pool, rows, kv_new, draft, accept_len, next_token):
    """In-place append of each sequence's committed entries at its length (arrays are modified)."""
    L, two, N, H, cap_pool, Dh = kv_pool.shape
    B = kv_new.shape[2]
    D = kv_new.shape[4] - 1
    assert kv_pool.flags.c_contiguous and len_pool.dtype == np.int32 and len_pool.flags.c_contiguous
    assert tok_pool is None or (tok_pool.dtype == np.int32 and tok_pool.flags.c_contiguous)
    _check(lib().oracle_append(L, H, Dh, kv_pool.dtype.itemsize, N, cap_pool, kv_pool.ctypes.data, _p(tok_pool),
                               _p(len_pool), _p(_i32(rows)), B, D,
                               np.ascontiguousarray(kv_new, dtype=kv_pool.dtype).ctypes.data,
                               _p(_i32(draft).reshape(-1)), _p(_i32(accept_len)), _p(_i32(next_token))))


# ----------------------------------------------------------------- paged KV

class PagedState:
    """A paged KV cache held in numpy arrays, operated on by the oracle's paged
    functions.  pages [L,2,n_pages,H,page,Dh]; bt [rows,max_blocks] (-1 = none);
    free [n_pages] stack with n_free entries; tokens [rows, max_blocks*page];
    len [rows]."""

    def __init__(self, L, H, Dh, n_pages, page, max_blocks, rows, dtype=np.float16, free_order=None):
        self.pages = np.zeros((L, 2, n_pages, H, page, Dh), dtype)
        self.bt = np.full((rows, max_blocks), -1, np.int32)
        self.free = (np.arange(n_pages, dtype=np.int32) if free_order is None
                     else np.ascontiguousarray(free_order, dtype=np.int32))
        self.n_free = np.array([n_pages], np.int32)
        self.tokens = np.zeros((rows, max_blocks * page), np.int32)
        self.len = np.zeros(rows, np.int32)
        self.geo = np.array([L, H, Dh, self.pages.itemsize, n_pages, page, max_blocks, rows], np.int32)

    def copy(self):
        c = PagedState.__new__(PagedState)
        for k in ("pages", "bt", "free", "n_free", "tokens", "len", "geo"):
            setattr(c, k, getattr(self, k).copy())
        return c


def _paged_lib():
    L = lib()
    if not hasattr(L, "_paged_ready"):
        vp, i32p, i8p, ci = C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int8), C.c_int
        L.oracle_paged_append.argtypes = [i32p, vp, i32p, i32p, i32p, i32p, i32p, i32p, ci, ci, vp, i32p, i32p, i32p,
                                          C.c_int32, i32p, i32p, i32p, i8p, ci]
        L.oracle_paged_gather.argtypes = [i32p, vp, i32p, i32p, i32p, i32p, ci, ci, vp, i32p, i32p, i8p, i32p, i32p,
                                          C.c_int32]
        L.oracle_paged_admit.argtypes = [i32p, vp, i32p, i32p, i32p, i32p, i32p, i32p, ci, vp, i32p, i32p, ci, ci]
        L.oracle_paged_retire.argtypes = [i32p, i32p, i32p, i32p, i32p, i32p, ci]
        for f in (L.oracle_paged_append, L.oracle_paged_gather, L.oracle_paged_admit, L.oracle_paged_retire):
            f.restype = C.c_int
        L._paged_ready = True
    return L


def paged_append(st, kv_new, draft, accept_len, next_token, rows=None, pad_token=0, rect_cap=None):
    """One round's realignment on the paged cache `st` (modified in place).
    Returns dict(width, tokens, pos, mask) with the [B, rect_cap] rectangle view
    (rect_cap defaults to the pool's row capacity)."""
    L_, two, B, H, D1, Dh = kv_new.shape
    D = D1 - 1
    rows = None if rows is None else _i32(rows)
    rect_cap = st.tokens.shape[1] if rect_cap is None else rect_cap
    tok = np.zeros((B, rect_cap), np.int32)
    pos = np.zeros((B, rect_cap), np.int32)
    mask = np.zeros((B, rect_cap), np.int8)
    width = np.zeros(1, np.int32)
    kv_new = np.ascontiguousarray(kv_new, dtype=st.pages.dtype)
    rc = _paged_lib().oracle_paged_append(_p(st.geo), st.pages.ctypes.data, _p(st.bt), _p(st.free), _p(st.n_free),
                                          _p(st.tokens), _p(st.len), _p(rows), B, D, kv_new.ctypes.data,
                                          _p(_i32(draft).reshape(-1)), _p(_i32(accept_len)), _p(_i32(next_token)),
                                          pad_token, _p(width), _p(tok), _p(pos), _p(mask, C.c_int8), rect_cap)
    _check(rc)
    W = int(width[0])
    return dict(width=W, tokens=tok[:, :W], pos=pos[:, :W], mask=mask[:, :W])


def paged_gather(st, rows=None, B=None, cap_out=None, pad_token=0):
    """The batch's rows as a left-padded rectangle: dict(kv, tokens, pos, mask, len, width)."""
    rows = None if rows is None else _i32(rows)
    B = (len(rows) if rows is not None else st.len.shape[0]) if B is None else B
    L_, _, _, H, _, Dh = st.pages.shape
    cap_out = st.tokens.shape[1] if cap_out is None else cap_out
    kv = np.zeros((L_, 2, B, H, cap_out, Dh), st.pages.dtype)
    tok = np.zeros((B, cap_out), np.int32)
    pos = np.zeros((B, cap_out), np.int32)
    mask = np.zeros((B, cap_out), np.int8)
    ln = np.zeros(B, np.int32)
    width = np.zeros(1, np.int32)
    rc = _paged_lib().oracle_paged_gather(_p(st.geo), st.pages.ctypes.data, _p(st.bt), _p(st.tokens), _p(st.len),
                                          _p(rows), B, cap_out, kv.ctypes.data, _p(tok), _p(pos),
                                          _p(mask, C.c_int8), _p(ln), _p(width), pad_token)
    _check(rc)
    W = int(width[0])
    return dict(kv=kv[..., :W, :], tokens=tok[:, :W], pos=pos[:, :W], mask=mask[:, :W], len=ln, width=W)


def paged_admit(st, in_kv, in_tok, in_len, S, rows=None):
    """Rows rows[b] (empty) receive the content of a left-padded rectangle of width S."""
    L_, _, B, H, cap_in, Dh = in_kv.shape
    rows = None if rows is None else _i32(rows)
    in_kv = np.ascontiguousarray(in_kv, dtype=st.pages.dtype)
    _check(_paged_lib().oracle_paged_admit(_p(st.geo), st.pages.ctypes.data, _p(st.bt), _p(st.free), _p(st.n_free),
                                           _p(st.tokens), _p(st.len), _p(rows), B, in_kv.ctypes.data,
                                           _p(_i32(in_tok).reshape(-1)), _p(_i32(in_len)), int(S), cap_in))


def paged_retire(st, rows):
    rows = _i32(rows)
    _check(_paged_lib().oracle_paged_retire(_p(st.geo), _p(st.bt), _p(st.free), _p(st.n_free), _p(st.len), _p(rows),
                                            len(rows)))


# ------------------------------------------------------------ pool lifecycle

class Sched:
    """Scheduling state of a pool of `slots` sequences: active [slots] slot ids in
    schedule order (n_active of them), free [slots] free slot ids ascending
    (n_free of them), q_head: the next queued prompt."""

    def __init__(self, slots, active=None):
        self.slots = slots
        self.active = np.zeros(slots, np.int32)
        self.free = np.zeros(slots, np.int32)
        act = list(range(slots)) if active is None else list(active)
        self.active[:len(act)] = act
        fr = [s for s in range(slots) if s not in set(act)]
        self.free[:len(fr)] = fr
        self.n_active = np.array([len(act)], np.int32)
        self.n_free = np.array([len(fr)], np.int32)
        self.q_head = np.zeros(1, np.int32)

    def copy(self):
        c = Sched.__new__(Sched)
        c.slots = self.slots
        for k in ("active", "free", "n_active", "n_free", "q_head"):
            setattr(c, k, getattr(self, k).copy())
        return c

    def active_list(self):
        return self.active[:int(self.n_active[0])].copy()

    def free_list(self):
        return self.free[:int(self.n_free[0])].copy()


def _pool_lib():
    L = lib()
    if not hasattr(L, "_pool_ready"):
        vp, i32p, ci = C.c_void_p, C.POINTER(C.c_int32), C.c_int
        L.oracle_pool_finish.argtypes = [i32p, ci, i32p, ci, i32p, i32p, i32p, i32p, i32p, i32p, ci, ci, C.c_int32,
                                         C.c_int32, i32p, i32p]
        L.oracle_pool_admit.argtypes = [ci, ci, ci, ci, vp, i32p, ci, i32p, ci, i32p, i32p, i32p, i32p, i32p, ci, vp,
                                        i32p, i32p, ci, i32p, i32p]
        L.oracle_pool_finish.restype = C.c_int
        L.oracle_pool_admit.restype = C.c_int
        L._pool_ready = True
    return L


def pool_finish(tok_pool, len_pool, sched, rows, accept_len, D, eos_id, max_len):
    """Finish at end-of-sequence or max length after a round's append (arrays and
    `sched` are modified); returns the retired slots in active-list order."""
    N, cap = tok_pool.shape
    assert tok_pool.dtype == np.int32 and tok_pool.flags.c_contiguous and len_pool.dtype == np.int32
    rows = _i32(rows)
    retired = np.zeros(N, np.int32)
    nr = np.zeros(1, np.int32)
    _check(_pool_lib().oracle_pool_finish(_p(tok_pool), cap, _p(len_pool), N, _p(sched.active), _p(sched.n_active),
                                          _p(sched.free), _p(sched.n_free), _p(rows), _p(_i32(accept_len)),
                                          rows.shape[0], D, eos_id, max_len, _p(retired), _p(nr)))
    return retired[:int(nr[0])]


def pool_admit(kv_pool, tok_pool, len_pool, sched, pkv, ptok, plen):
    """Admit queued prompts into the lowest free slots (arrays and `sched` are
    modified); returns the slots filled, in admission order."""
    L, _, N, H, cap, Dh = kv_pool.shape
    Q, pcap = ptok.shape
    assert kv_pool.flags.c_contiguous and tok_pool.flags.c_contiguous
    admitted = np.zeros(N, np.int32)
    na = np.zeros(1, np.int32)
    pkv = np.ascontiguousarray(pkv, dtype=kv_pool.dtype)
    _check(_pool_lib().oracle_pool_admit(L, H, Dh, kv_pool.dtype.itemsize, kv_pool.ctypes.data, _p(tok_pool), cap,
                                         _p(len_pool), N, _p(sched.active), _p(sched.n_active), _p(sched.free),
                                         _p(sched.n_free), _p(sched.q_head), Q, pkv.ctypes.data,
                                         _p(_i32(ptok)), _p(_i32(plen)), pcap, _p(admitted), _p(na)))
    return admitted[:int(na[0])]
