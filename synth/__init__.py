"""Seeded synthetic inputs shared by the oracle side and the GPU side.

Holds no step of the verify or realign computation: it only produces logits,
drafts, KV entries, lengths and uniforms, each a pure function of
(seed, stream, round, index) defined once in gen_core.h.
"""
import ctypes as C
import os

import numpy as np

from .configs import CONFIGS, Config, F32, F16, BF16, ESIZE, DTYPE_NAME  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
S_LEN, S_KV0, S_TOK0, S_LOGIT, S_PLANT, S_KVNEW, S_UNIF, S_NOISE = 1, 2, 3, 4, 5, 6, 7, 8

_host = None
_dev = None


def _i32p(a):
    return a.ctypes.data_as(C.POINTER(C.c_int32)) if a is not None else None


def host_lib():
    global _host
    if _host is None:
        path = os.path.join(HERE, "libsynth_host.so")
        if not os.path.exists(path):
            from . import _build
            _build.build_host()
        lib = C.CDLL(path)
        u64, u32, i64, f32, vp = C.c_uint64, C.c_uint32, C.c_int64, C.c_float, C.c_void_p
        i32p = C.POINTER(C.c_int32)
        lib.synth_fill_normal.argtypes = [C.c_int, u64, u32, u32, u64, u64, f32, vp]
        lib.synth_fill_uniform.argtypes = [u64, u32, u32, u64, u64, C.POINTER(C.c_float)]
        lib.synth_fill_int.argtypes = [u64, u32, u32, u64, u64, i64, i64, i32p]
        lib.synth_pool_lengths.argtypes = [u64, C.c_int, C.c_int, C.c_int, C.c_int, i32p]
        lib.synth_plan_greedy.argtypes = [u64, u32, C.c_int, C.c_int, C.c_int, C.c_int, C.c_double, C.c_double,
                                          i32p, i32p, i32p]
        lib.synth_fill_logits.argtypes = [C.c_int, u64, u32, i64, i64, i64, i64, f32, i32p, f32, vp]
        lib.synth_fill_kv.argtypes = [C.c_int, u64, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, i32p, C.c_int,
                                      C.c_int, C.c_int, C.c_int, vp]
        lib.synth_fill_tokens.argtypes = [u64, C.c_int, C.c_int, C.c_int, i32p, C.c_int, C.c_int, C.c_int32,
                                          i32p, i32p, C.POINTER(C.c_int8)]
        _host = lib
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        path = os.path.join(HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError("libsynth_dev.so is not built; run __graft_entry__.build()")
        lib = C.CDLL(path)
        u64, u32, i64, f32, vp = C.c_uint64, C.c_uint32, C.c_int64, C.c_float, C.c_void_p
        lib.synth_dev_fill_normal.argtypes = [C.c_int, u64, u32, u32, u64, u64, f32, vp, vp]
        lib.synth_dev_fill_logits.argtypes = [C.c_int, u64, u32, i64, i64, i64, i64, f32, vp, f32, vp, vp]
        lib.synth_dev_fill_kv.argtypes = [C.c_int, u64, C.c_int, C.c_int, C.c_int, C.c_int, vp, C.c_int, C.c_int,
                                          C.c_int, C.c_int, vp, vp]
        _dev = lib
    return _dev


def np_dtype(dt):
    return {F32: np.float32, F16: np.float16, BF16: np.uint16}[dt]


# ---------------------------------------------------------------- small tables

def lengths(cfg: Config) -> np.ndarray:
    """Initial content length of every row (pool sequence)."""
    if cfg.fixed_lens is not None:
        return np.array(cfg.fixed_lens, dtype=np.int32)
    out = np.empty(cfg.B, dtype=np.int32)
    if cfg.pool_values:
        rc = host_lib().synth_pool_lengths(cfg.seed, cfg.B, cfg.pool_values, cfg.len_lo, cfg.len_hi, _i32p(out))
        if rc != 0:
            raise ValueError("bad pool length recipe")
    else:
        host_lib().synth_fill_int(cfg.seed, S_LEN, 0, 0, cfg.B, cfg.len_lo, cfg.len_hi, _i32p(out))
    return out


def plan_greedy(cfg: Config, rnd: int, B=None):
    """(plant [B*(D+1),3], first_miss [B], draft [B,D]) of a greedy round."""
    B = cfg.B if B is None else B
    plant = np.empty((B * cfg.D1, 3), dtype=np.int32)
    miss = np.empty(B, dtype=np.int32)
    draft = np.empty((B, cfg.D), dtype=np.int32)
    host_lib().synth_plan_greedy(cfg.seed, rnd, B, cfg.D, cfg.V, cfg.plan_mode, cfg.plan_p, cfg.tie_frac,
                                 _i32p(plant), _i32p(miss), _i32p(draft))
    return plant, miss, draft


def uniforms(seed, stream, rnd, n, start=0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    host_lib().synth_fill_uniform(seed, stream, rnd, start, n, out.ctypes.data_as(C.POINTER(C.c_float)))
    return out


def normals(dtype, seed, stream, rnd, n, sigma=1.0, start=0) -> np.ndarray:
    out = np.empty(n, dtype=np_dtype(dtype))
    host_lib().synth_fill_normal(dtype, seed, stream, rnd, start, n, sigma, out.ctypes.data)
    return out


# ---------------------------------------------------------------- host tensors

def logits_host(cfg: Config, rnd: int, plant, row0=0, nrows=None, row_stride=None, V=None, sigma=None,
                dtype=None):
    """Logit rows [row0, row0+nrows) of round rnd as a [nrows, row_stride] array."""
    V = cfg.V if V is None else V
    nrows = plant.shape[0] - row0 if nrows is None else nrows
    stride = V if row_stride is None else row_stride
    dt = cfg.logit_dtype if dtype is None else dtype
    sg = cfg.sigma if sigma is None else sigma
    out = np.zeros((nrows, stride), dtype=np_dtype(dt))
    host_lib().synth_fill_logits(dt, cfg.seed, rnd, row0, nrows, V, stride, sg,
                                 _i32p(np.ascontiguousarray(plant, dtype=np.int32)) if plant is not None else None,
                                 cfg.plant_value, out.ctypes.data)
    return out


def kv_host(cfg: Config, lens, width, left_pad, layer0=0, nlayers=None, rows=None, cap=None):
    """KV buffer [nlayers,2,rows,H,cap,Dh] holding the initial content of layers layer0.."""
    nlayers = cfg.L if nlayers is None else nlayers
    rows = cfg.B if rows is None else rows
    cap = cfg.cap if cap is None else cap
    out = np.empty((nlayers, 2, rows, cfg.H, cap, cfg.Dh), dtype=np_dtype(cfg.kv_dtype))
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    host_lib().synth_fill_kv(cfg.kv_dtype, cfg.seed, cfg.L, rows, cfg.H, cap, cfg.Dh, _i32p(lens), int(width),
                             int(left_pad), layer0, nlayers, out.ctypes.data)
    return out


def kvnew_host(cfg: Config, rnd: int, layer0=0, nlayers=None, B=None):
    """KV entries of the D+1 verified positions, [nlayers,2,B,H,D+1,Dh], layers layer0.."""
    nlayers = cfg.L if nlayers is None else nlayers
    B = cfg.B if B is None else B
    per_layer = 2 * B * cfg.H * cfg.D1 * cfg.Dh
    flat = normals(cfg.kv_dtype, cfg.seed, S_KVNEW, rnd, nlayers * per_layer, 1.0, start=layer0 * per_layer)
    return flat.reshape(nlayers, 2, B, cfg.H, cfg.D1, cfg.Dh)


def tokens_host(cfg: Config, lens, width, left_pad, pad_token=0, rows=None, cap=None):
    rows = len(lens) if rows is None else rows
    cap = cfg.cap if cap is None else cap
    tok = np.empty((rows, cap), dtype=np.int32)
    pos = np.empty((rows, cap), dtype=np.int32)
    mask = np.empty((rows, cap), dtype=np.int8)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    host_lib().synth_fill_tokens(cfg.seed, rows, cap, cfg.V, _i32p(lens), int(width), int(left_pad), pad_token,
                                 _i32p(tok), _i32p(pos), mask.ctypes.data_as(C.POINTER(C.c_int8)))
    return tok, pos, mask


def sampled_logits_round(cfg: Config, rnd: int = 0, B=None, V=None):
    """The logits behind sampled_round: target logits ~ N(0, sigma) and draft
    logits = target + N(0, noise), both rounded once to float32, with the same
    draft ids and uniforms as sampled_round.  Returns target [B,D+1,V],
    draft_logits [B,D,V], draft [B,D], u_accept [B,D], u_draw [B,D+1]."""
    B = cfg.B if B is None else B
    V = cfg.V if V is None else V
    D, D1 = cfg.D, cfg.D1
    tl = normals(F32, cfg.seed, S_LOGIT, rnd, B * D1 * V, cfg.sigma).reshape(B, D1, V).astype(np.float64)
    noise = normals(F32, cfg.seed, S_NOISE, rnd, B * D * V, cfg.draft_noise).reshape(B, D, V).astype(np.float64)
    dl = tl[:, :D, :] + noise
    _, _, draft, u_acc, u_draw = sampled_round(cfg, rnd, B=B, V=V)
    return tl.astype(np.float32), dl.astype(np.float32), draft, u_acc, u_draw


def sampled_round(cfg: Config, rnd: int = 0, B=None, V=None):
    """Inputs of a sampled-verification round.

    Target logits ~ N(0, sigma), draft logits = target + N(0, noise); p and q are
    softmax(logits / temperature) evaluated in float64 and rounded to float32 once,
    so both sides read the same bytes.  Draft ids are drawn from q by numpy's
    seeded sampler (the draft model's own sampling, outside the verify step).
    Returns p [B,D+1,V], q [B,D,V], draft [B,D], u_accept [B,D], u_draw [B,D+1].
    """
    B = cfg.B if B is None else B
    V = cfg.V if V is None else V
    D, D1 = cfg.D, cfg.D1
    tl = normals(F32, cfg.seed, S_LOGIT, rnd, B * D1 * V, cfg.sigma).reshape(B, D1, V).astype(np.float64)
    noise = normals(F32, cfg.seed, S_NOISE, rnd, B * D * V, cfg.draft_noise).reshape(B, D, V).astype(np.float64)
    dl = tl[:, :D, :] + noise

    def softmax(x):
        z = x / cfg.temperature
        z = z - z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=-1, keepdims=True)

    p = softmax(tl).astype(np.float32)
    q = softmax(dl).astype(np.float32)
    rng = np.random.Generator(np.random.PCG64(cfg.seed * 1000003 + rnd))
    draft = np.empty((B, D), dtype=np.int32)
    for b in range(B):
        for i in range(D):
            qq = q[b, i].astype(np.float64)
            draft[b, i] = rng.choice(V, p=qq / qq.sum())
    u_acc = uniforms(cfg.seed, S_UNIF, rnd, B * D).reshape(B, D)
    u_draw = uniforms(cfg.seed, S_UNIF, rnd, B * D1, start=1 << 32).reshape(B, D1)
    return p, q, draft, u_acc, u_draw
