"""Determinism and stream behaviour of the C ABI on the GPU: identical inputs
give identical bytes, and independent calls enqueued on two streams give the
same results as the same calls run one after the other."""
import numpy as np
import pytest
import torch

import synth
import synth.device as sdev
from tests.gpu_util import say, to_np_raw

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_kv_realignment_amd as m
    return m


def _round(sd, w, bufs, r, ws):
    acc, nxt = sd.verify_greedy(w.logits[r], w.drafts[r], ws=ws)
    sd.realign_eqspec(bufs[0], bufs[1], w.kv_new[r], w.drafts[r], acc, nxt)
    return acc, nxt


def test_repeat_is_bit_identical(sd):
    """The 7b-mha round (fp32 logits, fp16 KV) run twice from the same state."""
    cfg = synth.CONFIGS["7b-mha"]
    say("determinism 7b-mha")
    w = sdev.GreedyRounds(cfg, 1)
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    bufs = [sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, tdt) for _ in range(2)]
    w.load_initial(bufs[0])
    ws = sd.workspace(cfg.B, cfg.D)
    outs = []
    for rep in range(2):
        bufs[1].kv.view(torch.uint8).fill_(rep + 1)
        acc, nxt = _round(sd, w, bufs, 0, ws)
        torch.cuda.synchronize()
        W = int(bufs[1].width.item())
        outs.append((acc.cpu().numpy(), nxt.cpu().numpy(), to_np_raw(bufs[1].kv[..., :W, :]),
                     bufs[1].tokens.cpu().numpy()[:, :W]))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def test_two_streams(sd):
    """Two independent batches (tiny and 7b-mha shapes) verified and realigned on
    two torch streams at once, compared with the same calls run serially."""
    say("two streams")
    results = {}
    for mode in ("serial", "streams"):
        setups = []
        for name in ("tiny", "7b-mha"):
            cfg = synth.CONFIGS[name]
            w = sdev.GreedyRounds(cfg, 1)
            tdt = sdev.TORCH_DT[cfg.kv_dtype]
            bufs = [sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, tdt) for _ in range(2)]
            w.load_initial(bufs[0])
            bufs[1].kv.zero_()
            setups.append((name, w, bufs, sd.workspace(cfg.B, cfg.D)))
        torch.cuda.synchronize()
        outs = {}
        if mode == "serial":
            for name, w, bufs, ws in setups:
                outs[name] = _round(sd, w, bufs, 0, ws)
        else:
            streams = [torch.cuda.Stream() for _ in setups]
            for (name, w, bufs, ws), st in zip(setups, streams):
                with torch.cuda.stream(st):
                    outs[name] = _round(sd, w, bufs, 0, ws)
            for st in streams:
                st.synchronize()
        torch.cuda.synchronize()
        results[mode] = {name: (outs[name][0].cpu().numpy(), outs[name][1].cpu().numpy(),
                                to_np_raw(bufs[1].kv[..., :int(bufs[1].width.item()), :]))
                         for name, w, bufs, ws in setups}
    for name in results["serial"]:
        for a, b in zip(results["serial"][name], results["streams"][name]):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), name
