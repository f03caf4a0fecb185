"""An empty batch through every entry point: no error, nothing written."""
import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_kv_realignment_amd as m
    return m


L, H, Dh, CAP, D, V = 2, 2, 8, 16, 3, 50


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32, device="cuda")


def _snapshot(*ts):
    return [t.clone() for t in ts]


def _same(before, *ts):
    """Byte equality: the buffers come from torch.empty, whose garbage may hold
    NaN patterns that a float comparison would call different from themselves."""
    return all(torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
               for a, b in zip(before, ts))


def test_empty_verification(sd):
    say("empty verification")
    status = _i32(1)
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        acc, nxt = sd.verify_greedy(torch.zeros((0, D + 1, V), dtype=dt, device="cuda"), _i32(0, D), status=status)
        assert acc.numel() == 0 and nxt.numel() == 0
        acc, nxt = sd.verify_sample_logits(torch.zeros((0, D + 1, V), dtype=dt, device="cuda"),
                                           torch.zeros((0, D, V), dtype=dt, device="cuda"), _i32(0, D),
                                           torch.zeros((0, D), device="cuda"), torch.zeros((0, D + 1), device="cuda"),
                                           0.8, top_p=0.9, status=status)
        assert acc.numel() == 0 and nxt.numel() == 0
    acc, nxt = sd.verify_sample(torch.zeros((0, D + 1, V), device="cuda"), torch.zeros((0, D, V), device="cuda"),
                                _i32(0, D), torch.zeros((0, D), device="cuda"), torch.zeros((0, D + 1), device="cuda"),
                                status=status)
    torch.cuda.synchronize()
    assert acc.numel() == 0 and int(status.item()) == 0


def test_empty_realignment(sd):
    say("empty realignment")
    status = _i32(1)
    kv_new = torch.zeros((L, 2, 0, H, D + 1, Dh), dtype=torch.float16, device="cuda")
    src = sd.SeqBuf.empty(L, 0, H, CAP, Dh, torch.float16)
    dst = sd.SeqBuf.empty(L, 0, H, CAP, Dh, torch.float16)
    dst.width.fill_(5)
    sd.realign_eqspec(src, dst, kv_new, _i32(0, D), _i32(0), _i32(0), status=status)
    sd.realign_eqspec_inplace(src, kv_new, _i32(0, D), _i32(0), _i32(0), status=status)
    # a pool of 3 rows: an empty append and an empty gather leave it as it was
    pool = sd.SeqBuf.empty(L, 3, H, CAP, Dh, torch.float16, pool=True)
    pool.kv.fill_(1.5)
    pool.len.copy_(torch.tensor([4, 0, 7], dtype=torch.int32))
    before = _snapshot(pool.kv, pool.tokens, pool.len)
    sd.append(pool, kv_new, _i32(0, D), _i32(0), _i32(0), rows=_i32(0), status=status)
    rect = sd.SeqBuf.empty(L, 3, H, CAP, Dh, torch.float16, groups=1)
    rect_before = _snapshot(rect.kv, rect.tokens, rect.width)
    sd.gather(pool, rect, _i32(0), 8, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(dst.width.item()) == 5
    assert _same(before, pool.kv, pool.tokens, pool.len) and _same(rect_before, rect.kv, rect.tokens, rect.width)


def test_empty_paged_and_pool_calls(sd):
    say("empty paged and pool calls")
    status = _i32(1)
    cache = sd.PagedKV.empty(L, 3, H, Dh, 6, 4, 2, torch.float16)
    before = _snapshot(cache.pages, cache.block_table, cache.free_pages, cache.n_free, cache.tokens, cache.len,
                       cache.sync)
    kv_new = torch.zeros((L, 2, 0, H, D + 1, Dh), dtype=torch.float16, device="cuda")
    sd.paged_append(cache, kv_new, _i32(0, D), _i32(0), _i32(0), rows=_i32(0), status=status)
    sd.paged_gather(cache, sd.SeqBuf.empty(L, 0, H, CAP, Dh, torch.float16), status=status)
    sd.paged_admit(cache, sd.SeqBuf.empty(L, 0, H, CAP, Dh, torch.float16), status=status)
    sd.paged_retire(cache, _i32(0), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert _same(before, cache.pages, cache.block_table, cache.free_pages, cache.n_free, cache.tokens, cache.len,
                 cache.sync)
    # admitting from an empty queue admits nothing and leaves the pool as it was
    pool = sd.SeqBuf.empty(L, 4, H, CAP, Dh, torch.float16, pool=True)
    sched = sd.Sched(4, active=[2, 0])
    pbefore = _snapshot(pool.kv, pool.tokens, pool.len, sched.active, sched.n_active, sched.free_slots,
                        sched.n_free, sched.q_head)
    adm, nadm = sd.pool_admit(pool, sched, sd.SeqBuf.empty(L, 0, H, CAP, Dh, torch.float16), status=status)
    torch.cuda.synchronize()
    assert int(nadm.item()) == 0 and int(status.item()) == 0
    assert _same(pbefore, pool.kv, pool.tokens, pool.len, sched.active, sched.n_active, sched.free_slots,
                 sched.n_free, sched.q_head)
