"""Pins of the oracle's realignment and grouping: invariants, the batched run
against the per-sequence brute force, closed forms of the generated workloads,
and mutation tests showing the checks catch the ragged-batch bug."""
import numpy as np
import pytest

import oracle
import synth
from oracle import brute
from tests import invariants as inv


def _random_rect(rng, B, D, L, H, Dh, cap, dtype=np.float32, pad_token=0):
    lens = rng.integers(0, cap - D - 1, B).astype(np.int32)
    if B:
        lens[rng.integers(0, B)] = max(1, int(lens.max()))
    S = int(lens.max()) if B else 0
    kv = np.zeros((L, 2, B, H, cap, Dh), dtype)
    tok = np.full((B, cap), pad_token, np.int32)
    mask = np.zeros((B, cap), np.int8)
    for b in range(B):
        pad = S - lens[b]
        kv[:, :, b, :, pad:S] = rng.standard_normal((L, 2, H, lens[b], Dh)).astype(dtype)
        tok[b, pad:S] = rng.integers(1, 1000, lens[b])
        mask[b, pad:S] = 1
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(dtype)
    acc = rng.integers(0, D + 1, B).astype(np.int32)
    draft = rng.integers(1, 1000, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 1000, B).astype(np.int32)
    return lens, S, kv, tok, mask, kv_new, acc, draft, nxt


@pytest.mark.parametrize("seed", range(40))
def test_eqspec_batched_equals_per_sequence_brute_force(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    D = int(rng.integers(0, 6))
    L, H, Dh = int(rng.integers(1, 3)), int(rng.integers(1, 3)), 4
    cap = 24
    dtype = [np.float32, np.float16][seed % 2]
    lens, S, kv, tok, mask, kv_new, acc, draft, nxt = _random_rect(rng, B, D, L, H, Dh, cap, dtype)
    out = oracle.realign_eqspec(kv, kv_new, lens, S, tok, mask, acc, nxt, draft)
    W = out["width"]
    committed = [list(draft[b, :acc[b]]) + [int(nxt[b])] for b in range(B)]
    inv.check_round(tok, mask, S, out["tokens"], out["pos"], out["mask"], out["len"], W, acc, committed, D)
    inv.check_kv_round(kv, lens, S, out["kv"], out["len"], W, kv_new, acc)
    for b in range(B):
        t0 = list(tok[b, S - lens[b]:S])
        kv0 = kv[:, :, b, :, S - lens[b]:S]
        t1, kv1 = brute.advance(t0, kv0, committed[b], kv_new[:, :, b])
        c1 = len(t1)
        assert list(out["tokens"][b, W - c1:W]) == t1
        assert np.array_equal(out["kv"][:, :, b, :, W - c1:W].view(np.uint8), kv1.view(np.uint8))
    # positions at and beyond the new width are not written
    assert np.all(out["kv"][:, :, :, :, W:] == 0)


def test_eqspec_rejects_inconsistent_inputs():
    rng = np.random.default_rng(1)
    lens, S, kv, tok, mask, kv_new, acc, draft, nxt = _random_rect(rng, 3, 4, 1, 1, 4, 16)
    bad = mask.copy()
    bad[0, S - 1] = 0
    with pytest.raises(oracle.OracleError):
        oracle.realign_eqspec(kv, kv_new, lens, S, tok, bad, acc, nxt, draft)
    with pytest.raises(oracle.OracleError):
        oracle.realign_eqspec(kv, kv_new, lens, S, tok, mask, np.array([5, 0, 0]), nxt, draft)
    with pytest.raises(oracle.OracleError) as e:
        oracle.realign_eqspec(kv, kv_new, lens, S, tok, mask, acc, nxt, draft, cap_out=int(lens.max()))
    assert e.value.code == oracle.E_CAPACITY


def test_tiny_workload_batched_equals_unbatched():
    """The tiny workload: one greedy cycle on the batch of two equals two unbatched cycles."""
    cfg = synth.CONFIGS["tiny"]
    lens = synth.lengths(cfg)
    S = int(lens.max())
    plant, miss, draft = synth.plan_greedy(cfg, 0)
    logits = synth.logits_host(cfg, 0, plant)
    kv = synth.kv_host(cfg, lens, S, True)
    kv_new = synth.kvnew_host(cfg, 0)
    tok, pos, mask = synth.tokens_host(cfg, lens, S, True)
    acc, nxt, _ = oracle.verify_greedy(logits, draft, cfg.B, cfg.D, cfg.V)
    assert np.array_equal(acc, miss)  # planted closed form
    out = oracle.realign_eqspec(kv, kv_new, lens, S, tok, mask, acc, nxt, draft)
    W = out["width"]
    for b in range(cfg.B):
        a, committed = brute.greedy_one(logits[b * cfg.D1:(b + 1) * cfg.D1], draft[b])
        t1, kv1 = brute.advance(list(tok[b, S - lens[b]:S]), kv[:, :, b, :, S - lens[b]:S], committed,
                                kv_new[:, :, b])
        c1 = len(t1)
        assert out["len"][b] == c1
        assert list(out["tokens"][b, W - c1:W]) == t1
        assert np.array_equal(out["kv"][:, :, b, :, W - c1:W], kv1)
        assert list(out["pos"][b, W - c1:W]) == list(range(c1))


@pytest.mark.parametrize("name,rounds", [("tiny", 1), ("7b-mha", 3), ("8b-gqa", 2)])
def test_generated_rounds_accept_planted_length(name, rounds):
    """Closed form of the generated workloads: the plan puts a value above every
    other logit at its designed id (ties only at higher ids), so the accepted
    length equals the plan's first mismatching position and the next token is the
    designed id of that row."""
    cfg = synth.CONFIGS[name]
    for r in range(rounds):
        plant, miss, draft = synth.plan_greedy(cfg, r)
        logits = synth.logits_host(cfg, r, plant)
        acc, nxt, tgt = oracle.verify_greedy(logits, draft, cfg.B, cfg.D, cfg.V)
        assert np.array_equal(acc, miss)
        assert np.array_equal(tgt.reshape(-1), plant[:, 0])
        assert np.array_equal(nxt, plant.reshape(cfg.B, cfg.D1, 3)[np.arange(cfg.B), acc, 0])


# -------------------------------------------------------------- grouping

def test_group_by_len_hand_example():
    # lengths by id: 0:5 1:3 2:5 3:5 4:3 5:7, batches of 2
    # (length, id) order: 1,4 | 0,2,3 | 5 ; full batches: [1,4] (3) [0,2] (5); leftovers 3, 5
    order, uni, wid, nu = oracle.group_by_len([5, 3, 5, 5, 3, 7], 2)
    assert list(order) == [1, 4, 0, 2, 3, 5]
    assert list(uni) == [1, 1, 0]
    assert list(wid) == [3, 5, 7]
    assert nu == 2


@pytest.mark.parametrize("seed", range(30))
def test_group_by_len_invariants(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(0, 70))
    G = int(rng.integers(1, 9))
    lens = rng.integers(1, 6, N).astype(np.int32)
    order, uni, wid, nu = oracle.group_by_len(lens, G)
    assert sorted(order.tolist()) == list(range(N))
    full_expected = sum(int(c) // G for c in np.bincount(lens)) if N else 0
    nb = (N + G - 1) // G
    assert len(uni) == nb
    for g in range(nb):
        grp = lens[order[g * G:(g + 1) * G]]
        assert uni[g] == int(grp.min() == grp.max())
        assert wid[g] == grp.max()
    # the leading batches are the full same-length ones, ascending length
    lead = [lens[order[g * G]] for g in range(full_expected)]
    assert all(uni[g] for g in range(full_expected))
    assert lead == sorted(lead)
    assert nu >= full_expected
    assert nu == int(np.sum(uni))


def test_pool_workload_first_round_is_all_uniform():
    cfg = synth.CONFIGS["exspec"]
    lens = synth.lengths(cfg)
    assert len(np.unique(lens)) == cfg.pool_values
    order, uni, wid, nu = oracle.group_by_len(lens, cfg.group)
    assert nu == cfg.B // cfg.group and np.all(uni == 1)


def test_gather_append_pool_round():
    """One pool round: mixed batches gathered into left-padded rectangles, then
    every sequence appends its committed entries in place."""
    rng = np.random.default_rng(5)
    N, G, D, L, H, Dh, cap = 12, 4, 3, 2, 1, 4, 20
    lens = rng.integers(1, 10, N).astype(np.int32)
    lens[:4] = 6
    kv = np.zeros((L, 2, N, H, cap, Dh), np.float32)
    tok = np.zeros((N, cap), np.int32)
    for r in range(N):
        kv[:, :, r, :, :lens[r]] = rng.standard_normal((L, 2, H, lens[r], Dh))
        tok[r, :lens[r]] = rng.integers(1, 100, lens[r])
    order, uni, wid, nu = oracle.group_by_len(lens, G)
    rect_cap = 16
    out = oracle.gather(kv, tok, lens, order, G, uni, rect_cap)
    for g in range(len(uni)):
        rows = order[g * G:(g + 1) * G]
        if uni[g]:
            assert np.all(out["mask"][g * G:(g + 1) * G] == 0)  # untouched
            continue
        W = int(out["width"][g])
        assert W == lens[rows].max()
        inv.check_rect(out["tokens"][g * G:(g + 1) * G], out["pos"][g * G:(g + 1) * G],
                       out["mask"][g * G:(g + 1) * G], lens[rows], W)
        for k, r in enumerate(rows):
            j = g * G + k
            assert np.array_equal(out["kv"][:, :, j, :, W - lens[r]:W], kv[:, :, r, :, :lens[r]])
            assert np.array_equal(out["tokens"][j, W - lens[r]:W], tok[r, :lens[r]])
    kv_new = rng.standard_normal((L, 2, N, H, D + 1, Dh)).astype(np.float32)
    acc = rng.integers(0, D + 1, N).astype(np.int32)
    draft = rng.integers(1, 100, (N, D)).astype(np.int32)
    nxt = rng.integers(1, 100, N).astype(np.int32)
    kv2, tok2, len2 = kv.copy(), tok.copy(), lens.copy()
    oracle.append(kv2, tok2, len2, np.arange(N), kv_new, draft, acc, nxt)
    for r in range(N):
        committed = list(draft[r, :acc[r]]) + [int(nxt[r])]
        t1, k1 = brute.advance(list(tok[r, :lens[r]]), kv[:, :, r, :, :lens[r]], committed, kv_new[:, :, r])
        assert len2[r] == len(t1)
        assert list(tok2[r, :len2[r]]) == t1
        assert np.array_equal(kv2[:, :, r, :, :len2[r]], k1)
    with pytest.raises(oracle.OracleError):
        oracle.append(kv2, tok2, len2, np.array([0, 0]), kv_new[:, :, :2], draft, acc, nxt)


# -------------------------------------------------------------- mutations

def _one_round(seed=3):
    rng = np.random.default_rng(seed)
    B, D = 5, 4
    while True:
        lens, S, kv, tok, mask, kv_new, acc, draft, nxt = _random_rect(rng, B, D, 1, 2, 4, 24)
        if len(set(acc.tolist())) > 1:
            break
    out = oracle.realign_eqspec(kv, kv_new, lens, S, tok, mask, acc, nxt, draft)
    committed = [list(draft[b, :acc[b]]) + [int(nxt[b])] for b in range(B)]
    return lens, S, kv, tok, mask, kv_new, acc, draft, nxt, out, committed, D


def test_checker_accepts_correct_round():
    lens, S, kv, tok, mask, kv_new, acc, draft, nxt, out, committed, D = _one_round()
    inv.check_round(tok, mask, S, out["tokens"], out["pos"], out["mask"], out["len"], out["width"], acc, committed, D)
    inv.check_kv_round(kv, lens, S, out["kv"], out["len"], out["width"], kv_new, acc)


def test_checker_rejects_ragged_append_without_repad():
    """The ragged-tensor bug: every row appends its committed tokens after column
    S with no repad, so rows end at different columns."""
    lens, S, kv, tok, mask, kv_new, acc, draft, nxt, out, committed, D = _one_round()
    B = len(lens)
    t2, m2 = tok.copy(), mask.copy()
    for b in range(B):
        n = len(committed[b])
        t2[b, S:S + n] = committed[b]
        m2[b, S:S + n] = 1
    W = S + max(len(c) for c in committed)
    pos2 = np.zeros_like(t2)
    for b in range(B):
        pos2[b, :W] = np.maximum(np.cumsum(m2[b, :W]) - 1, 0)
    with pytest.raises(inv.InvariantError):
        inv.check_round(tok, mask, S, t2, pos2, m2, out["len"], W, acc, committed, D)


def test_checker_rejects_uniform_shift():
    """Every row shifted by the batch's largest commit count instead of its own:
    rows that committed fewer tokens end before the rectangle's last column."""
    lens, S, kv, tok, mask, kv_new, acc, draft, nxt, out, committed, D = _one_round()
    B = len(lens)
    n_max = max(len(c) for c in committed)
    W = S + n_max
    t2 = np.zeros((B, W), np.int32)
    m2 = np.zeros((B, W), np.int8)
    for b in range(B):
        c, n = int(lens[b]), len(committed[b])
        start = W - c - n_max
        t2[b, start:start + c] = tok[b, S - c:S]
        t2[b, start + c:start + c + n] = committed[b]
        m2[b, start:start + c + n] = 1
    pos2 = np.where(m2 == 1, np.cumsum(m2, axis=1) - 1, 0)
    with pytest.raises(inv.InvariantError):
        inv.check_round(tok, mask, S, t2, pos2, m2, out["len"], W, acc, committed, D)


def test_checker_rejects_dropped_bonus():
    lens, S, kv, tok, mask, kv_new, acc, draft, nxt, out, committed, D = _one_round()
    short = [c[:-1] for c in committed]
    with pytest.raises(inv.InvariantError):
        inv.check_round(tok, mask, S, out["tokens"], out["pos"], out["mask"], out["len"], out["width"], acc, short, D)


def test_checker_rejects_off_by_one_positions():
    lens, S, kv, tok, mask, kv_new, acc, draft, nxt, out, committed, D = _one_round()
    pos = out["pos"] + out["mask"]
    with pytest.raises(inv.InvariantError):
        inv.check_round(tok, mask, S, out["tokens"], pos, out["mask"], out["len"], out["width"], acc, committed, D)


def test_checker_rejects_unshifted_kv():
    """Tokens realigned but the KV cache left at its old columns."""
    lens, S, kv, tok, mask, kv_new, acc, draft, nxt, out, committed, D = _one_round()
    kv2 = out["kv"].copy()
    kv2[..., :S, :] = kv[..., :S, :]
    with pytest.raises(inv.InvariantError):
        inv.check_kv_round(kv, lens, S, kv2, out["len"], out["width"], kv_new, acc)


@pytest.mark.parametrize("seed", range(12))
def test_chain_final_equals_batched_oracle_chain(seed):
    """The per-sequence chain model (brute.chain_final) equals the batched oracle
    applied round after round, on random chains of 1-9 rounds; the pool layout
    equals oracle.append applied round after round."""
    rng = np.random.default_rng(900 + seed)
    B, D = int(rng.integers(1, 7)), int(rng.integers(0, 5))
    L, H, Dh = int(rng.integers(1, 3)), int(rng.integers(1, 3)), 4
    R = int(rng.integers(1, 10))
    cap = 20 + R * (D + 1)
    dtype = [np.float32, np.float16][seed % 2]
    lens, S, kv, tok, mask, _, _, draft, nxt = _random_rect(rng, B, D, L, H, Dh, 20, dtype)
    kv = np.concatenate([kv, np.zeros((L, 2, B, H, cap - 20, Dh), dtype)], axis=4)
    tok = np.concatenate([tok, np.zeros((B, cap - 20), np.int32)], axis=1)
    mask = np.concatenate([mask, np.zeros((B, cap - 20), np.int8)], axis=1)
    news = [rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(dtype) for _ in range(R)]
    accs = [rng.integers(0, D + 1, B).astype(np.int32) for _ in range(R)]
    want, want_lens, W = brute.chain_final(kv, lens, S, news, accs)
    cur, cl, cS, ct, cm = kv, lens, S, tok, mask
    for r in range(R):
        out = oracle.realign_eqspec(cur, news[r], cl, cS, ct, cm, accs[r], nxt, draft)
        cur, cl, cS, ct, cm = out["kv"], out["len"], out["width"], out["tokens"], out["mask"]
    assert cS == W and np.array_equal(cl, want_lens)
    assert np.array_equal(cur[..., :W, :].view(np.uint8), want.view(np.uint8))
    # pool layout: rows left-aligned, appended in place
    pool = np.zeros((L, 2, B, H, cap, Dh), dtype)
    for b in range(B):
        pool[:, :, b, :, :lens[b]] = kv[:, :, b, :, S - lens[b]:S]
    ptok, plen = np.zeros((B, cap), np.int32), lens.copy()
    for r in range(R):
        oracle.append(pool, ptok, plen, np.arange(B), news[r], draft, accs[r], nxt)
    pw, plens, PW = brute.chain_final(pool, lens, 0, news, accs, left_pad=False)
    assert np.array_equal(plens, plen) and PW == W
    assert np.array_equal(pool[..., :PW, :].view(np.uint8), pw.view(np.uint8))
