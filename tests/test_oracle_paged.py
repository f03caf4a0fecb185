"""Pins of the oracle's paged KV functions (block tables, the realignment as
metadata): a paged chain gathered back into a rectangle equals the EQSPEC
oracle's chain byte for byte; a per-row list model gives the same content;
pages stay a partition of the pool; admit/gather/retire round trips; capacity
errors change nothing."""
import numpy as np
import pytest

import oracle
from oracle import brute
from tests.test_oracle_realign import _random_rect


def _pages_partition(st):
    """Every page is either free or in exactly one row's table, and each row
    holds exactly ceil(len / page) pages."""
    n_pages, page = st.pages.shape[2], st.pages.shape[4]
    nf = int(st.n_free[0])
    used = [int(x) for x in st.bt.reshape(-1) if x >= 0]
    allp = sorted(list(st.free[:nf]) + used)
    assert allp == list(range(n_pages))
    for r in range(st.bt.shape[0]):
        nb = -(-int(st.len[r]) // page)
        assert np.all(st.bt[r, :nb] >= 0) and np.all(st.bt[r, nb:] == -1)


def _new_state(rng, L, H, Dh, B, page, max_blocks, spare, dtype):
    n_pages = B * max_blocks + spare
    return oracle.PagedState(L, H, Dh, n_pages, page, max_blocks, B, dtype,
                             free_order=rng.permutation(n_pages).astype(np.int32))


@pytest.mark.parametrize("seed", range(24))
def test_paged_chain_equals_eqspec_chain(seed):
    """admit a left-padded rectangle, then several rounds of paged append; after
    each round the gathered rectangle equals the EQSPEC oracle's output."""
    rng = np.random.default_rng(300 + seed)
    B = int(rng.integers(1, 6))
    D = int(rng.integers(0, 5))
    L, H, Dh = int(rng.integers(1, 3)), int(rng.integers(1, 3)), 4
    page = int(rng.choice([1, 2, 3, 4, 8]))
    rounds = 4
    cap = 16 + rounds * (D + 1)
    dtype = [np.float32, np.float16][seed % 2]
    lens, S, kv, tok, mask, _, _, _, _ = _random_rect(rng, B, D, L, H, Dh, 16, dtype)
    kv = np.concatenate([kv, np.zeros(kv.shape[:4] + (cap - 16, Dh), dtype)], axis=4)
    tok = np.concatenate([tok, np.zeros((B, cap - 16), np.int32)], axis=1)
    mask = np.concatenate([mask, np.zeros((B, cap - 16), np.int8)], axis=1)
    st = _new_state(rng, L, H, Dh, B, page, -(-cap // page), int(rng.integers(0, 3)), dtype)
    oracle.paged_admit(st, kv, tok, lens, S)
    _pages_partition(st)
    g = oracle.paged_gather(st, cap_out=cap)
    assert g["width"] == S and np.array_equal(g["len"], lens)
    assert np.array_equal(g["kv"].view(np.uint8), kv[..., :S, :].view(np.uint8))
    assert np.array_equal(g["tokens"], tok[:, :S]) and np.array_equal(g["mask"], mask[:, :S])
    cur = dict(kv=kv, tokens=tok, mask=mask, len=lens, width=S)
    for r in range(rounds):
        kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(dtype)
        acc = rng.integers(0, D + 1, B).astype(np.int32)
        draft = rng.integers(1, 1000, (B, D)).astype(np.int32)
        nxt = rng.integers(1, 1000, B).astype(np.int32)
        want = oracle.realign_eqspec(cur["kv"], kv_new, cur["len"], cur["width"], cur["tokens"], cur["mask"], acc,
                                     nxt, draft, cap_out=cap)
        view = oracle.paged_append(st, kv_new, draft, acc, nxt, rect_cap=cap)
        _pages_partition(st)
        W = want["width"]
        assert view["width"] == W
        assert np.array_equal(view["tokens"], want["tokens"][:, :W])
        assert np.array_equal(view["pos"], want["pos"][:, :W])
        assert np.array_equal(view["mask"], want["mask"][:, :W])
        g = oracle.paged_gather(st, cap_out=cap)
        assert g["width"] == W and np.array_equal(g["len"], want["len"])
        assert np.array_equal(g["kv"].view(np.uint8), want["kv"][..., :W, :].view(np.uint8))
        assert np.array_equal(g["tokens"], want["tokens"][:, :W]) and np.array_equal(g["pos"], want["pos"][:, :W])
        cur = want


def test_paged_append_matches_per_row_list_model():
    """The paged content of every row equals the per-sequence brute force
    (old content, then the committed tokens and the first n speculative entries)."""
    rng = np.random.default_rng(7)
    B, D, L, H, Dh, page = 5, 3, 2, 2, 4, 3
    st = _new_state(rng, L, H, Dh, B, page, 8, 4, np.float32)
    rows = np.array([3, 0, 4], np.int32)  # a batch of pool rows, not all rows
    lens = np.array([5, 0, 7], np.int32)
    S = 7
    kv = np.zeros((L, 2, 3, H, S, Dh), np.float32)
    tok = np.zeros((3, S), np.int32)
    for b in range(3):
        kv[:, :, b, :, S - lens[b]:] = rng.standard_normal((L, 2, H, lens[b], Dh))
        tok[b, S - lens[b]:] = rng.integers(1, 99, lens[b])
    oracle.paged_admit(st, kv, tok, lens, S, rows=rows)
    model = [(list(tok[b, S - lens[b]:]), kv[:, :, b, :, S - lens[b]:]) for b in range(3)]
    for _ in range(3):
        kv_new = rng.standard_normal((L, 2, 3, H, D + 1, Dh)).astype(np.float32)
        acc = rng.integers(0, D + 1, 3).astype(np.int32)
        draft = rng.integers(1, 99, (3, D)).astype(np.int32)
        nxt = rng.integers(1, 99, 3).astype(np.int32)
        oracle.paged_append(st, kv_new, draft, acc, nxt, rows=rows)
        model = [brute.advance(t, k, list(draft[b, :acc[b]]) + [int(nxt[b])], kv_new[:, :, b])
                 for b, (t, k) in enumerate(model)]
        _pages_partition(st)
    g = oracle.paged_gather(st, rows=rows)
    W = g["width"]
    for b, (t, k) in enumerate(model):
        c = len(t)
        assert int(st.len[rows[b]]) == c
        assert list(g["tokens"][b, W - c:]) == t
        assert np.array_equal(g["kv"][:, :, b, :, W - c:], k)
        assert np.all(g["kv"][:, :, b, :, :W - c] == 0)
    # rows outside the batch stay empty
    assert st.len[1] == 0 and st.len[2] == 0 and np.all(st.bt[[1, 2]] == -1)


def test_paged_append_moves_only_committed_entries():
    """Pages already holding content are not rewritten: bytes outside the
    committed slots are unchanged."""
    rng = np.random.default_rng(8)
    B, D, L, H, Dh, page = 3, 4, 1, 2, 4, 4
    st = _new_state(rng, L, H, Dh, B, page, 6, 2, np.float32)
    lens = np.array([6, 9, 1], np.int32)
    S = 9
    kv = rng.standard_normal((L, 2, B, H, S, Dh)).astype(np.float32)
    oracle.paged_admit(st, kv, np.ones((B, S), np.int32), lens, S)
    before = st.pages.copy()
    bt0, len0 = st.bt.copy(), st.len.copy()
    acc = np.array([4, 0, 2], np.int32)
    oracle.paged_append(st, np.ones((L, 2, B, H, D + 1, Dh), np.float32), np.zeros((B, D), np.int32), acc,
                        np.zeros(B, np.int32))
    changed = np.any(before != st.pages, axis=(0, 1, 3, 5))  # [n_pages, page]
    expect = np.zeros_like(changed)
    for b in range(B):
        for j in range(len0[b], len0[b] + acc[b] + 1):
            expect[st.bt[b, j // page], j % page] = True
    assert np.array_equal(changed, expect)
    assert np.array_equal(st.bt[bt0 >= 0], bt0[bt0 >= 0])  # existing blocks keep their pages


def test_paged_capacity_errors_change_nothing():
    rng = np.random.default_rng(9)
    B, D, page = 2, 3, 2
    st = oracle.PagedState(1, 1, 4, 5, page, 3, B, np.float32)
    lens = np.array([4, 3], np.int32)
    kv = rng.standard_normal((1, 2, B, 1, 4, 4)).astype(np.float32)
    oracle.paged_admit(st, kv, np.ones((B, 4), np.int32), lens, 4)
    assert int(st.n_free[0]) == 1
    snap = st.copy()
    kv_new = np.zeros((1, 2, B, 1, D + 1, 4), np.float32)
    # row 0 grows 4 -> 6 (one new page) and row 1 grows 3 -> 5 (one new page): two needed, one free
    with pytest.raises(oracle.OracleError) as e:
        oracle.paged_append(st, kv_new, np.zeros((B, D), np.int32), np.array([1, 1], np.int32),
                            np.zeros(B, np.int32))
    assert e.value.code == oracle.E_CAPACITY
    # a row past max_blocks * page positions
    with pytest.raises(oracle.OracleError) as e:
        oracle.paged_append(st, kv_new, np.zeros((B, D), np.int32), np.array([3, 0], np.int32),
                            np.zeros(B, np.int32))
    assert e.value.code == oracle.E_CAPACITY
    with pytest.raises(oracle.OracleError):  # accepted length outside [0, D]
        oracle.paged_append(st, kv_new, np.zeros((B, D), np.int32), np.array([0, 4], np.int32),
                            np.zeros(B, np.int32))
    with pytest.raises(oracle.OracleError):  # admitting into a row that is not empty
        oracle.paged_admit(st, kv, np.ones((B, 4), np.int32), lens, 4)
    for k in ("pages", "bt", "free", "n_free", "tokens", "len"):
        assert np.array_equal(getattr(st, k), getattr(snap, k)), k
    # one row alone fits
    oracle.paged_append(st, kv_new[:, :, :1], np.zeros((1, D), np.int32), np.array([1], np.int32),
                        np.zeros(1, np.int32), rows=[0])
    assert int(st.n_free[0]) == 0 and st.len[0] == 6
    _pages_partition(st)


def test_paged_retire_and_readmit():
    rng = np.random.default_rng(10)
    L, H, Dh, page, B = 1, 2, 4, 4, 4
    st = _new_state(rng, L, H, Dh, B, page, 4, 0, np.float16)
    lens = np.array([3, 16, 0, 9], np.int32)
    kv = rng.standard_normal((L, 2, B, H, 16, Dh)).astype(np.float16)
    tok = rng.integers(1, 50, (B, 16)).astype(np.int32)
    oracle.paged_admit(st, kv, tok, lens, 16)
    nf0 = int(st.n_free[0])
    pushed = list(st.bt[3, :3]) + list(st.bt[1, :4])
    oracle.paged_retire(st, [3, 1])
    _pages_partition(st)
    assert int(st.n_free[0]) == nf0 + 3 + 4 and st.len[1] == 0 and st.len[3] == 0
    # the retired rows' pages go back on the stack in block order, row 3 first
    assert list(st.free[nf0:nf0 + 7]) == pushed
    kv2 = rng.standard_normal((L, 2, 2, H, 16, Dh)).astype(np.float16)
    tok2 = rng.integers(1, 50, (2, 16)).astype(np.int32)
    oracle.paged_admit(st, kv2, tok2, np.array([16, 5], np.int32), 16, rows=[1, 3])
    _pages_partition(st)
    g = oracle.paged_gather(st, rows=[1, 3, 0])
    assert g["width"] == 16 and list(g["len"]) == [16, 5, 3]
    assert np.array_equal(g["kv"][:, :, 0], kv2[:, :, 0])
    assert np.array_equal(g["kv"][:, :, 1, :, 11:], kv2[:, :, 1, :, 11:])
    assert np.array_equal(g["kv"][:, :, 2, :, 13:], kv[:, :, 0, :, 13:])
    assert np.array_equal(g["tokens"][1, 11:], tok2[1, 11:])
