"""Device-resident workloads built from the seeded generator (set-up only).

Allocates torch device tensors and fills them with libsynth_dev, so multi-GB
KV caches and per-round logits never cross PCIe.  The values are exactly those
of the host functions in this package.
"""
import numpy as np
import torch

from . import (BF16, F16, F32, S_KVNEW, dev_lib, lengths, plan_greedy, tokens_host)

TORCH_DT = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ok(rc):
    if rc != 0:
        raise RuntimeError("device generator launch failed")


def fill_logits(cfg, rnd, plant, out, row0=0):
    """out: [..., V] device tensor of cfg's logit type holding rows row0.. of round rnd."""
    V = out.shape[-1]
    nrows = out.numel() // V
    plant_dev = torch.from_numpy(np.ascontiguousarray(plant, dtype=np.int32)).to(out.device)
    _ok(dev_lib().synth_dev_fill_logits(cfg.logit_dtype, cfg.seed, rnd, row0, nrows, V, V, cfg.sigma,
                                        plant_dev.data_ptr(), cfg.plant_value, out.data_ptr(), _stream()))
    return plant_dev  # keep alive until the stream has consumed it


def fill_normal(dtype, seed, stream, rnd, out, sigma=1.0, start=0):
    _ok(dev_lib().synth_dev_fill_normal(dtype, seed, stream, rnd, start, out.numel(), sigma, out.data_ptr(),
                                        _stream()))


def fill_kvnew(cfg, rnd, out, layer0=0):
    """out: [nl, 2, B, H, D+1, Dh] = the round's speculative KV of layers layer0.."""
    per_layer = out.numel() // out.shape[0]
    fill_normal(cfg.kv_dtype, cfg.seed, S_KVNEW, rnd, out, 1.0, start=layer0 * per_layer)


def fill_kv(cfg, kv, lens_dev, width, left_pad, layer0=0):
    """kv: [nl, 2, rows, H, cap, Dh] holding the initial content of layers layer0.."""
    nl, _, rows, H, cap, Dh = kv.shape
    _ok(dev_lib().synth_dev_fill_kv(cfg.kv_dtype, cfg.seed, rows, H, cap, Dh, lens_dev.data_ptr(), int(width),
                                    int(left_pad), layer0, nl, kv.data_ptr(), _stream()))


class GreedyRounds:
    """All inputs of `rounds` chained greedy rounds of a left-padded batch:
    logits [R, B, D+1, V], drafts [R, B, D], speculative KV [R, L, 2, B, H, D+1, Dh],
    plus the initial rectangle state as host arrays and device tensors."""

    def __init__(self, cfg, rounds, device="cuda", with_kvnew=True):
        self.cfg, self.rounds, self.device = cfg, rounds, device
        B, D1 = cfg.B, cfg.D1
        self.lens0 = lengths(cfg)
        self.width0 = int(self.lens0.max())
        self.plans = [plan_greedy(cfg, r) for r in range(rounds)]
        self.drafts = torch.from_numpy(np.stack([p[2] for p in self.plans])).to(device)
        self.logits = torch.empty((rounds, B, D1, cfg.V), dtype=TORCH_DT[cfg.logit_dtype], device=device)
        keep = []
        for r in range(rounds):
            keep.append(fill_logits(cfg, r, self.plans[r][0], self.logits[r]))
        self.kv_new = None
        if with_kvnew:
            self.kv_new = torch.empty((rounds, cfg.L, 2, B, cfg.H, D1, cfg.Dh), dtype=TORCH_DT[cfg.kv_dtype],
                                      device=device)
            for r in range(rounds):
                fill_kvnew(cfg, r, self.kv_new[r])
        torch.cuda.current_stream().synchronize()
        self.tok0, self.pos0, self.mask0 = tokens_host(cfg, self.lens0, self.width0, True)

    def load_initial(self, buf):
        """Write the initial left-padded state into SeqBuf `buf`."""
        lens_dev = torch.from_numpy(self.lens0).to(self.device)
        fill_kv(self.cfg, buf.kv, lens_dev, self.width0, True)
        tok, pos, mask = (self.tok0, self.pos0, self.mask0) if buf.cap == self.cfg.cap else \
            tokens_host(self.cfg, self.lens0, self.width0, True, cap=buf.cap)
        buf.tokens.copy_(torch.from_numpy(tok))
        buf.pos.copy_(torch.from_numpy(pos))
        buf.mask.copy_(torch.from_numpy(mask))
        buf.len.copy_(lens_dev)
        buf.width.fill_(self.width0)
