"""Every-layer checks of the final state of full-size chains (GPU tests).

The expected bytes of each layer come from the oracle, one layer at a time, on
inputs regenerated on the host: the per-sequence chain model
(oracle.brute.chain_final) for rectangles, oracle.append round after round for
the pool, the batched realignment and gather where one round is checked.  The
GPU layer is downloaded one at a time, so host memory stays at a few layers."""
import numpy as np
import torch

import oracle
import synth
from oracle import brute
from tests.gpu_util import bytes_equal, say, to_np_raw


def check_chain_final_layers(cfg, lens0, width0, acc_hist, gpu_layer, what, canary=None):
    """Every layer of a left-padded rectangle after the chain whose accepted
    lengths per round are acc_hist [R][B]: gpu_layer(l) is the device tensor of
    layer l [2, B, H, cap, Dh].  Positions [W, cap) must hold `canary` bytes
    when given.  Returns the final width."""
    W = None
    R = len(acc_hist)
    for l in range(cfg.L):
        say(what, "final state, layer", l)
        kv0 = synth.kv_host(cfg, lens0, width0, True, layer0=l, nlayers=1)
        news = [synth.kvnew_host(cfg, r, layer0=l, nlayers=1) for r in range(R)]
        want, lens, W = brute.chain_final(kv0, lens0, width0, news, acc_hist)
        g = to_np_raw(gpu_layer(l))
        assert bytes_equal(g[..., :W, :], want[0]), "%s: final layer %d" % (what, l)
        if canary is not None:
            assert np.all(g[..., W:, :].view(np.uint8) == canary), "%s: layer %d written past width" % (what, l)
    return W


def device_equal(dev_tensor, host_array):
    """Byte equality of a device tensor and a host array of the same shape,
    compared on the device (the expected bytes are uploaded)."""
    a = dev_tensor.contiguous().view(torch.uint8).reshape(-1)
    b = torch.from_numpy(np.ascontiguousarray(host_array).view(np.uint8).reshape(-1)).to(dev_tensor.device)
    return a.numel() == b.numel() and bool(torch.equal(a, b))
