"""Greedy verification with the library's static workspace
(specdec_verify_greedy_noalloc), called through the C ABI: its results equal
those of specdec_verify_greedy with a caller workspace, bit for bit, on two
calls in a row (the second smaller), and it allocates nothing."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sdev
from tests.gpu_util import from_np_raw, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_kv_realignment_amd as m
    return m


def _outputs(B, D):
    return (torch.full((B,), -5, dtype=torch.int32, device="cuda"),
            torch.full((B,), -5, dtype=torch.int32, device="cuda"),
            torch.full((B, D + 1), -5, dtype=torch.int32, device="cuda"),
            torch.zeros(1, dtype=torch.int32, device="cuda"))


def _both(sd, logits, dt, row_stride, B, D, V, draft):
    """(no-alloc results, caller-workspace results), each (accept, next, target, status) on the host."""
    L = sd.lib()
    stream = torch.cuda.current_stream().cuda_stream
    acc, nxt, tgt, st = _outputs(B, D)
    before = torch.cuda.memory_allocated()
    rc = L.specdec_verify_greedy_noalloc(logits.data_ptr(), dt, row_stride, B, D, V, draft.data_ptr(),
                                         acc.data_ptr(), nxt.data_ptr(), tgt.data_ptr(), st.data_ptr(), stream)
    assert rc == sd.specdec.OK
    assert torch.cuda.memory_allocated() == before
    ws = sd.workspace(B, D, logits.device)
    acc2, nxt2, tgt2, st2 = _outputs(B, D)
    rc = L.specdec_verify_greedy(logits.data_ptr(), dt, row_stride, B, D, V, draft.data_ptr(), acc2.data_ptr(),
                                 nxt2.data_ptr(), tgt2.data_ptr(), ws.data_ptr(), ws.numel(), st2.data_ptr(), stream)
    assert rc == sd.specdec.OK
    torch.cuda.synchronize()
    host = lambda *ts: tuple(t.cpu().numpy() for t in ts)  # noqa: E731
    return host(acc, nxt, tgt, st), host(acc2, nxt2, tgt2, st2)


def _same(a, b):
    return all(np.array_equal(x, y) for x, y in zip(a, b))


def test_noalloc_equals_caller_workspace_twice(sd):
    # call 1: a full-size round of the 8b-gqa workload (B=16, D=5, V=151936 bf16)
    cfg = synth.CONFIGS["8b-gqa"]
    say("noalloc call 1", cfg.name, cfg.B, cfg.D, cfg.V)
    w = sdev.GreedyRounds(cfg, 1, with_kvnew=False)
    logits = w.logits[0]
    draft = w.drafts[0].contiguous()
    got, ref = _both(sd, logits, sd.BF16, cfg.V, cfg.B, cfg.D, cfg.V, draft)
    assert _same(got, ref)
    plant, _, hdraft = w.plans[0]
    oacc, onxt, otgt = oracle.verify_greedy(synth.logits_host(cfg, 0, plant), hdraft, cfg.B, cfg.D, cfg.V)
    assert np.array_equal(got[0], oacc) and np.array_equal(got[1], onxt) and np.array_equal(got[2], otgt)
    assert int(got[3][0]) == 0
    del w, logits

    # call 2: smaller (B=3, D=2, V=1000 fp32), strided rows, ties at the maximum
    B, D, V, rs = 3, 2, 1000, 1040
    say("noalloc call 2", B, D, V, rs)
    rng = np.random.default_rng(11)
    rows = rng.integers(-4, 4, size=(B * (D + 1), V)).astype(np.float32)
    rows[:, 997] = 4.0
    rows[:, 13] = 4.0                     # ties: the lower id wins
    buf = np.zeros((B * (D + 1), rs), np.float32)
    buf[:, :V] = rows
    dev = from_np_raw(buf.reshape(-1), torch.float32)
    logits = torch.as_strided(dev, (B, D + 1, V), (rs * (D + 1), rs, 1))
    hdraft = np.array([[13, 13], [13, 5], [7, 13]], np.int32)
    draft = torch.from_numpy(hdraft).cuda()
    got, ref = _both(sd, logits, sd.F32, rs, B, D, V, draft)
    assert _same(got, ref)
    oacc, onxt, otgt = oracle.verify_greedy(buf, hdraft, B, D, V, row_stride=rs)
    assert list(oacc) == [2, 1, 0]
    assert np.array_equal(got[0], oacc) and np.array_equal(got[1], onxt) and np.array_equal(got[2], otgt)


def test_noalloc_limits(sd):
    L = sd.lib()
    say("noalloc limits")
    x = torch.zeros(8, dtype=torch.float32, device="cuda")
    o = torch.zeros(8, dtype=torch.int32, device="cuda")
    p = x.data_ptr()
    # B * (D + 2) lines of 128 bytes must fit the 4 MiB array: 32768 lines
    assert L.specdec_verify_greedy_noalloc(p, sd.F32, 1, 16385, 0, 1, None, p, p, None, None, None) == \
        sd.specdec.E_SCRATCH
    assert L.specdec_verify_greedy_noalloc(p, sd.F32, 1, 0, 0, 1, None, None, None, None, None, None) == sd.specdec.OK
    assert L.specdec_verify_greedy_noalloc(p, 7, 1, 1, 0, 1, None, p, p, None, None, None) == sd.specdec.E_DTYPE
    # the largest batch that fits, B = 16384 at D = 0, runs and agrees with the caller-workspace call
    B, V = 16384, 3
    say("noalloc at the limit", B, V)
    rng = np.random.default_rng(3)
    rows = rng.integers(0, 3, size=(B, V)).astype(np.float32)
    logits = from_np_raw(rows.reshape(-1), torch.float32).view(B, 1, V)
    draft = torch.empty((B, 0), dtype=torch.int32, device="cuda")
    got, ref = _both(sd, logits, sd.F32, V, B, 0, V, draft)
    assert _same(got, ref)
    assert np.array_equal(got[1], rows.argmax(axis=1).astype(np.int32))
    del x, o
