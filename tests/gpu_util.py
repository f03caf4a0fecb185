"""Helpers for the GPU parity tests: device/host transfers of raw KV bytes."""
import sys

import numpy as np
import torch


def say(*a):
    """Name the case before a GPU step, flushed, so a failing run shows where it was."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def to_np_raw(t):
    """Device tensor -> host numpy array with the same element bytes (bf16 as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_np_raw(a, dtype, device="cuda"):
    """Host numpy array (bf16 as uint16 bits) -> device tensor of `dtype`."""
    a = np.ascontiguousarray(a)
    if dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device=device, dtype=dtype)


def bytes_equal(a, b):
    return a.shape == b.shape and np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                                                 np.ascontiguousarray(b).view(np.uint8))
