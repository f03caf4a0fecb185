"""The OpenMP build of the oracle (used only to time it on all host cores)
computes the same bytes as the single-threaded build the other tests pin."""
import numpy as np
import pytest

import oracle
from tests.test_oracle_realign import _random_rect


@pytest.fixture
def threaded():
    oracle.use_threads(True)
    try:
        yield
    finally:
        oracle.use_threads(False)


def _both(fn):
    oracle.use_threads(False)
    one = fn()
    oracle.use_threads(True)
    many = fn()
    return one, many


def test_threaded_build_reports_threads(threaded):
    assert oracle.threads() >= 1
    oracle.use_threads(False)
    assert oracle.threads() == 1


@pytest.mark.parametrize("seed", range(6))
def test_greedy_same_with_threads(seed, threaded):
    rng = np.random.default_rng(seed)
    B, D, V = int(rng.integers(1, 40)), int(rng.integers(0, 6)), int(rng.integers(1, 300))
    logits = rng.integers(-4, 4, (B, D + 1, V)).astype(np.float32)  # many ties
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    one, many = _both(lambda: oracle.verify_greedy(logits, draft, B, D, V))
    for x, y in zip(one, many):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("seed", range(6))
def test_realign_same_with_threads(seed, threaded):
    rng = np.random.default_rng(100 + seed)
    B, D = int(rng.integers(1, 9)), int(rng.integers(0, 5))
    L, H, Dh, cap = int(rng.integers(1, 4)), int(rng.integers(1, 4)), 8, 40
    lens, S, kv, tok, mask, kvn, acc, draft, nxt = _random_rect(rng, B, D, L, H, Dh, cap, np.float16)
    one, many = _both(lambda: oracle.realign_eqspec(kv, kvn, lens, S, tok, mask, acc, nxt, draft))
    assert one["width"] == many["width"]
    for k in ("kv", "tokens", "pos", "mask", "len"):
        np.testing.assert_array_equal(one[k].view(np.uint8), many[k].view(np.uint8))
