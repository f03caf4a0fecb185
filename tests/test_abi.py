"""The C-ABI library without a GPU: it loads, exports every entry point its
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re
import subprocess

import pytest

from ragged_kv_realignment_amd import specdec as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specdec.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(specdec_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_steps():
    names = _declared()
    for n in ("specdec_verify_greedy", "specdec_verify_sample", "specdec_realign_kv", "specdec_group_by_len"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = S.lib()
    for n in _declared():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (specdec_\w+)", out))
    assert set(_declared()) <= exported
    assert set(S.EXPORTS) == set(_declared())


def test_version_and_workspace_size():
    assert S.specdec_version().startswith("specdec")
    L = S.lib()
    assert L.specdec_workspace_bytes(16, 5) >= 16 * 6 * 8 + 16 * 4
    assert L.specdec_workspace_bytes(-1, 5) == 0
    # sizes the verification rejects report 0 instead of a wrapped byte count
    assert L.specdec_workspace_bytes(16, 256) == 0
    assert L.specdec_workspace_bytes(2**31 - 1, 2**31 - 1) == 0
    assert L.specdec_workspace_bytes(1 << 16, 255) == (1 << 16) * 257 * 128


FAKE = 0x10000  # never dereferenced: every call below fails validation on the host


def test_verify_greedy_host_errors():
    L = S.lib()
    f = L.specdec_verify_greedy
    ws_need = L.specdec_workspace_bytes(2, 3)
    args = dict(logits=FAKE, dt=S.BF16, rs=100, B=2, D=3, V=100, draft=FAKE, acc=FAKE, nxt=FAKE, tgt=None,
                ws=FAKE, wsb=ws_need, st=None, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["logits"], a["dt"], a["rs"], a["B"], a["D"], a["V"], a["draft"], a["acc"], a["nxt"], a["tgt"],
                 a["ws"], a["wsb"], a["st"], a["stream"])

    assert call(B=-1) == S.E_ARG
    assert call(D=-1) == S.E_ARG
    assert call(D=256) == S.E_ARG
    assert call(D=2**31 - 1) == S.E_ARG
    assert call(V=0) == S.E_ARG
    assert call(rs=99) == S.E_ARG
    assert call(dt=7) == S.E_DTYPE
    assert call(logits=None) == S.E_ARG
    assert call(draft=None) == S.E_ARG
    assert call(ws=None) == S.E_WORKSPACE
    assert call(wsb=ws_need - 1) == S.E_WORKSPACE
    assert call(ws=FAKE + 4) == S.E_WORKSPACE
    assert call(B=0) == S.OK  # empty batch: nothing to do


def test_verify_sample_host_errors():
    L = S.lib()
    f = L.specdec_verify_sample
    need = L.specdec_verify_sample_workspace_bytes(2, 2, 10)
    assert f(FAKE, FAKE, -1, 2, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None, None) == S.E_ARG
    assert f(FAKE, FAKE, 2, 2, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None, None) == S.E_ARG
    assert f(None, FAKE, 2, 2, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None, None) == S.E_ARG
    assert f(FAKE, None, 2, 2, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None, None) == S.E_ARG
    assert f(FAKE, FAKE, 2, 2, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None, None) == S.E_WORKSPACE
    assert f(FAKE, FAKE, 2, 2, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None, None) == S.E_WORKSPACE
    assert f(FAKE, FAKE, 2, 2, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, need, None, None) == S.E_WORKSPACE
    assert f(FAKE, FAKE, 2, 256, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None, None) == S.E_ARG   # D > 255
    assert f(FAKE, FAKE, 0, 2, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None) == S.OK


def test_verify_sample_workspace_size():
    L = S.lib()
    # a fixed block per row: a counter line, then 16 bytes for each of at most 16 splits and 16 x 256 runs
    row = 128 + 16 * 16 + 16 * 256 * 16
    assert L.specdec_verify_sample_workspace_bytes(32, 8, 32000) == 32 * row
    assert L.specdec_verify_sample_workspace_bytes(1, 0, 1) == row
    assert L.specdec_verify_sample_workspace_bytes(3, 2, 151936) == 3 * row
    assert L.specdec_verify_sample_workspace_bytes(-1, 2, 10) == 0
    assert L.specdec_verify_sample_workspace_bytes(1, 2, 0) == 0


def _sb(kv=FAKE, rows=4, cap=64, layers=2, heads=2, head_dim=128, dtype=S.BF16, tokens=FAKE, pos=FAKE, mask=FAKE,
        ln=FAKE, width=FAKE):
    return S.SeqBufC(kv, tokens, pos, mask, ln, width, rows, cap, layers, heads, head_dim, dtype)


def test_realign_host_errors():
    f = S.lib().specdec_realign_kv

    def call(mode, a, b, B=4, group=0, D=3, kv_new=FAKE * 100, rows=None, skip=None):
        return f(mode, C.byref(a), C.byref(b), rows, B, group, skip, D, kv_new, FAKE, FAKE, FAKE, 0, None, None)

    src = _sb(kv=FAKE * 1000)
    dst = _sb(kv=FAKE * 2000)
    assert call(9, src, dst) == S.E_ARG
    assert call(S.EQSPEC, src, dst, B=1025) == S.E_ARG
    assert call(S.EQSPEC, _sb(dtype=5), dst) == S.E_DTYPE
    assert call(S.EQSPEC, _sb(kv=FAKE * 1000, head_dim=4), _sb(kv=FAKE * 2000, head_dim=4)) == S.E_ALIGN
    assert call(S.EQSPEC, _sb(kv=FAKE * 1000 + 8), dst) == S.E_ALIGN
    assert call(S.EQSPEC, src, _sb(kv=FAKE * 2000, heads=3)) == S.E_ARG
    assert call(S.EQSPEC, src, _sb(kv=FAKE * 1000 + 4096)) == S.E_ALIAS       # KV ranges overlap
    assert call(S.EQSPEC, src, dst, B=3) == S.E_ARG                            # B != rows
    assert call(S.EQSPEC, src, _sb(kv=FAKE * 2000, width=None)) == S.E_ARG
    assert call(S.EQSPEC, src, dst, kv_new=FAKE * 100 + 8) == S.E_ALIGN
    assert call(S.GATHER, src, dst, group=0) == S.E_ARG
    assert call(S.GATHER, src, _sb(kv=FAKE * 2000, rows=3), group=2) == S.E_ARG
    assert call(S.APPEND_INPLACE, src, dst) == S.E_ARG                         # not the same pool
    assert call(S.APPEND_INPLACE, src, src, kv_new=None) == S.E_ARG
    # the largest draft counts are rejected, never wrapped into a small size
    assert call(5, src, src) == S.E_ARG
    assert call(S.EQSPEC_INPLACE_ZERO_PAD, src, dst) == S.E_ARG                # in place: the same buffers
    assert call(S.EQSPEC_INPLACE_ZERO_PAD, src, src, kv_new=None) == S.E_ARG
    for mode in (S.EQSPEC, S.EQSPEC_INPLACE, S.EQSPEC_INPLACE_ZERO_PAD, S.APPEND_INPLACE):
        assert call(mode, src, dst if mode == S.EQSPEC else src, D=2**31 - 1) == S.E_ARG
        assert call(mode, src, dst if mode == S.EQSPEC else src, D=2**27) == S.E_ARG


def test_group_by_len_host_errors():
    f = S.lib().specdec_group_by_len
    assert f(FAKE, -1, 8, FAKE, FAKE, FAKE, FAKE, None) == S.E_ARG
    assert f(FAKE, 4097, 8, FAKE, FAKE, FAKE, FAKE, None) == S.E_ARG
    assert f(FAKE, 16, 0, FAKE, FAKE, FAKE, FAKE, None) == S.E_ARG
    assert f(FAKE, 16, 8, None, FAKE, FAKE, FAKE, None) == S.E_ARG


def test_verify_greedy_noalloc_host_errors():
    """Rejected before any HIP call: the static scratch holds 32768 lines of 128 bytes."""
    f = S.lib().specdec_verify_greedy_noalloc
    assert f(FAKE, S.F32, 1, 16385, 0, 1, None, FAKE, FAKE, None, None, None) == S.E_SCRATCH
    assert f(FAKE, S.F32, 1, 2, 16383, 1, FAKE, FAKE, FAKE, None, None, None) == S.E_ARG   # D > 255
    assert f(FAKE, S.F32, 1, 5462, 4, 1, FAKE, FAKE, FAKE, None, None, None) == S.E_SCRATCH
    assert f(FAKE, S.F32, 1, -1, 4, 1, FAKE, FAKE, FAKE, None, None, None) == S.E_ARG
    assert f(FAKE, 9, 1, 1, 4, 1, FAKE, FAKE, FAKE, None, None, None) == S.E_DTYPE
    assert f(None, S.F32, 1, 1, 4, 1, FAKE, FAKE, FAKE, None, None, None) == S.E_ARG
    assert f(FAKE, S.F32, 1, 0, 4, 1, None, None, None, None, None, None) == S.OK   # empty batch: no-op


def test_workspace_init_null():
    assert S.lib().specdec_workspace_init(None, 256, None) == S.E_WORKSPACE


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(S, "_lib", None)
    monkeypatch.setattr(S, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError):
        S.lib()


def test_paged_and_pool_host_errors():
    """The paged-cache, lifecycle and sampling entry points reject bad arguments on
    the host (nothing here reaches a HIP call)."""
    L = S.lib()
    good = S.PagedC(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 8, 4, 2, 2, 64, S.BF16)
    kv_new = FAKE
    app = L.specdec_paged_append

    def call(c, **kw):
        a = dict(rows=None, B=2, D=3, kv_new=kv_new, draft=FAKE, acc=FAKE, nxt=FAKE, rect=None, cap=0)
        a.update(kw)
        return app(C.byref(c), a["rows"], a["B"], a["D"], a["kv_new"], a["draft"], a["acc"], a["nxt"], 0, None,
                   a["rect"], None, None, a["cap"], None, None)

    assert call(good, B=-1) == S.E_ARG
    assert call(good, B=1025) == S.E_ARG
    assert call(good, kv_new=None) == S.E_ARG
    assert call(good, kv_new=FAKE + 8) == S.E_ALIGN
    assert call(good, rect=FAKE, cap=0) == S.E_ARG
    bad = S.PagedC(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, 16, 8, 4, 2, 2, 64, S.BF16)  # no arrival counter
    assert call(bad) == S.E_ARG
    bad = S.PagedC(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 8, 4, 2, 2, 64, 7)
    assert call(bad) == S.E_DTYPE
    bad = S.PagedC(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 8, 4, 2, 2, 4, S.BF16)  # 8-byte positions
    assert call(bad) == S.E_ALIGN
    assert L.specdec_paged_retire(C.byref(good), FAKE, -1, None, None) == S.E_ARG
    # lifecycle: more than 4096 pool rows, bad max_len
    pool = S.SeqBufC(FAKE, FAKE, None, None, FAKE, None, 5000, 16, 2, 2, 64, S.BF16)
    sched = S.SchedC(FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.specdec_pool_finish(C.byref(pool), C.byref(sched), FAKE, FAKE, 1, 3, 2, 10, FAKE, FAKE, None,
                                 None) == S.E_ARG
    pool = S.SeqBufC(FAKE, FAKE, None, None, FAKE, None, 64, 16, 2, 2, 64, S.BF16)
    assert L.specdec_pool_finish(C.byref(pool), C.byref(sched), FAKE, FAKE, 1, 3, 2, 0, FAKE, FAKE, None,
                                 None) == S.E_ARG
    nos = S.SchedC(FAKE, None, FAKE, FAKE, FAKE)
    assert L.specdec_pool_admit(C.byref(pool), C.byref(nos), C.byref(pool), FAKE, FAKE, None, None) == S.E_ARG
    # grouping over pool rows needs the ids
    assert L.specdec_group_by_len_ids(FAKE, None, 8, 2, FAKE, FAKE, FAKE, FAKE, None) == S.E_ARG
    # sampled verification from logits: temperature and top-p ranges
    g = L.specdec_verify_sample_logits
    for T, tp in ((0.0, 1.0), (1.0, 0.0), (1.0, 1.5), (float("nan"), 1.0)):
        assert g(FAKE, FAKE, S.F32, 2, 3, 100, T, tp, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None,
                 None) == S.E_ARG
