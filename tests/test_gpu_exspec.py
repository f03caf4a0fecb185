"""GPU parity of equal-length scheduling: grouping, gather of mixed batches and
in-place append over the 256-sequence pool workload, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sdev
from tests import invariants as inv
from tests.full_layers import device_equal
from tests.gpu_util import bytes_equal, say, to_np_raw

pytestmark = pytest.mark.gpu

CANARY_KV = 0x5A
CANARY_I32 = -9


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_kv_realignment_amd as m
    return m


@pytest.mark.parametrize("seed", range(10))
def test_group_by_len_random(sd, seed):
    rng = np.random.default_rng(900 + seed)
    N = [0, 1, 7, 256, 1000, 4096, 300, 64, 513, 2048][seed]
    G = [1, 17, 4000][seed % 3] if seed in (1, 2, 7) else int(rng.integers(1, 17))
    lens = rng.integers(1, int(rng.integers(2, 40)), N).astype(np.int32)
    say("group_by_len", N, G)
    order, uni, wid, nu = sd.group_by_len(torch.from_numpy(lens).cuda(), G)
    torch.cuda.synchronize()
    oorder, ouni, owid, onu = oracle.group_by_len(lens, G)
    assert np.array_equal(order.cpu().numpy(), oorder)
    assert np.array_equal(uni.cpu().numpy(), ouni)
    assert np.array_equal(wid.cpu().numpy(), owid)
    assert int(nu.item()) == onu


@pytest.mark.parametrize("N,G,kind", [(777, 5, "wide"), (4096, 8, "equal"), (1024, 3, "wide"), (255, 16, "equal")])
def test_group_by_len_wide_values(sd, N, G, kind):
    """Lengths over the whole int32 range (negative ones included: ranked as
    signed integers) and pools of one length, against the oracle."""
    rng = np.random.default_rng(N + G)
    if kind == "wide":
        vals = rng.integers(-2**31, 2**31 - 1, 40, dtype=np.int64).astype(np.int32)
        vals[:3] = (-2**31, 2**31 - 1, 0)
        lens = vals[rng.integers(0, len(vals), N)]
    else:
        lens = np.full(N, 1234, np.int32)
    say("group_by_len", kind, N, G)
    order, uni, wid, nu = sd.group_by_len(torch.from_numpy(lens).cuda(), G)
    torch.cuda.synchronize()
    oorder, ouni, owid, onu = oracle.group_by_len(lens, G)
    assert np.array_equal(order.cpu().numpy(), oorder)
    assert np.array_equal(uni.cpu().numpy(), ouni)
    assert np.array_equal(wid.cpu().numpy(), owid)
    assert int(nu.item()) == onu


def test_group_by_len_host_errors(sd):
    say("group_by_len host errors")
    with pytest.raises(sd.SpecDecError):
        sd.group_by_len(torch.zeros(4097, dtype=torch.int32, device="cuda"), 8)
    with pytest.raises(sd.SpecDecError):
        sd.group_by_len(torch.zeros(8, dtype=torch.int32, device="cuda"), 0)


def test_gather_append_small(sd):
    """A small pool: gather of mixed groups (skipping uniform ones) and append,
    with canaries on everything that must stay untouched."""
    rng = np.random.default_rng(42)
    N, G, D, L, H, Dh, cap = 37, 4, 3, 2, 3, 8, 40
    lens = rng.integers(0, 20, N).astype(np.int32)
    lens[:8] = 11
    kv = np.zeros((L, 2, N, H, cap, Dh), np.float16)
    tok = np.full((N, cap), 0, np.int32)
    for r in range(N):
        kv[:, :, r, :, :lens[r]] = rng.standard_normal((L, 2, H, lens[r], Dh))
        tok[r, :lens[r]] = rng.integers(1, 100, lens[r])
    pool = sd.SeqBuf(torch.from_numpy(kv).cuda(), torch.from_numpy(tok).cuda(), torch.from_numpy(lens).cuda())
    order, uni, wid, nu = oracle.group_by_len(lens, G)
    rect_cap = 24
    rect = sd.SeqBuf.empty(L, N, H, rect_cap, Dh, torch.float16, groups=len(uni))
    rect.kv.view(torch.uint8).fill_(CANARY_KV)
    rect.tokens.fill_(CANARY_I32)
    rect.pos.fill_(CANARY_I32)
    rect.len.fill_(CANARY_I32)
    rect.width.fill_(CANARY_I32)
    say("gather small")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sd.gather(pool, rect, torch.from_numpy(order).cuda(), G, torch.from_numpy(uni).cuda(), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    want = oracle.gather(kv, tok, lens, order, G, uni, rect_cap)
    gk = to_np_raw(rect.kv)
    gt, gp, gm = rect.tokens.cpu().numpy(), rect.pos.cpu().numpy(), rect.mask.cpu().numpy()
    gw, gl = rect.width.cpu().numpy(), rect.len.cpu().numpy()
    for g in range(len(uni)):
        sl = slice(g * G, min(N, g * G + G))
        if uni[g]:
            assert np.all(gk[:, :, sl].view(np.uint8) == CANARY_KV) and np.all(gt[sl] == CANARY_I32)
            assert gw[g] == CANARY_I32
            continue
        W = want["width"][g]
        assert gw[g] == W
        assert bytes_equal(gk[:, :, sl, :, :W], want["kv"][:, :, sl, :, :W])
        assert np.all(gk[:, :, sl, :, W:].view(np.uint8) == CANARY_KV)
        for name, a in (("tokens", gt), ("pos", gp), ("mask", gm)):
            assert np.array_equal(a[sl, :W], want[name][sl, :W]), name
        assert np.array_equal(gl[sl], lens[order[sl]])
        inv.check_rect(gt[sl], gp[sl], gm[sl], lens[order[sl]], W)

    say("append small")
    kv_new = rng.standard_normal((L, 2, N, H, D + 1, Dh)).astype(np.float16)
    acc = rng.integers(0, D + 1, N).astype(np.int32)
    draft = rng.integers(1, 100, (N, D)).astype(np.int32)
    nxt = rng.integers(1, 100, N).astype(np.int32)
    sd.append(pool, torch.from_numpy(kv_new).cuda(), torch.from_numpy(draft).cuda(), torch.from_numpy(acc).cuda(),
              torch.from_numpy(nxt).cuda(), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    kv2, tok2, len2 = kv.copy(), tok.copy(), lens.copy()
    oracle.append(kv2, tok2, len2, np.arange(N), kv_new, draft, acc, nxt)
    assert np.array_equal(pool.len.cpu().numpy(), len2)
    assert np.array_equal(pool.tokens.cpu().numpy(), tok2)
    assert bytes_equal(to_np_raw(pool.kv), kv2)

    say("append capacity")
    full = torch.full((N,), cap, dtype=torch.int32, device="cuda")
    pool2 = sd.SeqBuf(pool.kv, pool.tokens, full)
    before = to_np_raw(pool.kv)
    status.zero_()
    sd.append(pool2, torch.from_numpy(kv_new).cuda(), torch.from_numpy(draft).cuda(), torch.from_numpy(acc).cuda(),
              torch.from_numpy(nxt).cuda(), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & sd.S_CAPACITY
    assert bytes_equal(to_np_raw(pool.kv), before)
    assert np.all(full.cpu().numpy() == cap)

    say("append duplicate rows")
    status.zero_()
    rows = torch.tensor([1, 1], dtype=torch.int32, device="cuda")
    sd.append(pool, torch.from_numpy(kv_new[:, :, :2].copy()).cuda(), torch.from_numpy(draft[:2].copy()).cuda(),
              torch.zeros(2, dtype=torch.int32, device="cuda"), torch.from_numpy(nxt[:2].copy()).cuda(), rows=rows,
              status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & sd.S_ROWS_DUP


@pytest.mark.parametrize("dup_at", [None, (0, 1023), (511, 512), (3, 900)])
def test_append_duplicate_rows_large_batch(sd, dup_at):
    """1,024 batch entries (the limit) naming distinct pool rows, or two of
    them naming the same row: the duplicate is found wherever it sits (status
    bit), and distinct rows never raise it (the append then matches the
    oracle)."""
    rng = np.random.default_rng(1300 if dup_at is None else 1300 + dup_at[0])
    rows_n, B, D, L, H, Dh, cap = 1100, 1024, 2, 1, 1, 8, 16
    lens = rng.integers(0, 10, rows_n).astype(np.int32)
    kv = rng.standard_normal((L, 2, rows_n, H, cap, Dh)).astype(np.float16)
    tok = rng.integers(1, 100, (rows_n, cap)).astype(np.int32)
    rows = rng.permutation(rows_n)[:B].astype(np.int32)
    if dup_at is not None:
        rows[dup_at[1]] = rows[dup_at[0]]
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float16)
    acc = rng.integers(0, D + 1, B).astype(np.int32)
    draft = rng.integers(1, 100, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 100, B).astype(np.int32)
    say("append dup large", dup_at)
    pool = sd.SeqBuf(torch.from_numpy(kv).cuda(), torch.from_numpy(tok).cuda(), torch.from_numpy(lens).cuda())
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sd.append(pool, torch.from_numpy(kv_new).cuda(), torch.from_numpy(draft).cuda(), torch.from_numpy(acc).cuda(),
              torch.from_numpy(nxt).cuda(), rows=torch.from_numpy(rows).cuda(), status=status)
    torch.cuda.synchronize()
    if dup_at is not None:
        assert int(status.item()) & sd.S_ROWS_DUP
        return
    assert int(status.item()) == 0
    wkv, wtok, wlen = kv.copy(), tok.copy(), lens.copy()
    oracle.append(wkv, wtok, wlen, rows, kv_new, draft, acc, nxt)
    assert bytes_equal(to_np_raw(pool.kv), wkv)
    assert np.array_equal(pool.tokens.cpu().numpy(), wtok)
    assert np.array_equal(pool.len.cpu().numpy(), wlen)


def test_exspec_pool_workload(sd):
    """The 256-sequence pool (40 layers x 2 KV heads x 128, bf16), 32 rounds:
    group by length, gather mixed batches, verify all rows, append in place."""
    cfg = synth.CONFIGS["exspec"]
    N, G, R = cfg.B, cfg.group, cfg.rounds
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    say("exspec setup")
    lens0 = synth.lengths(cfg)
    pool = sd.SeqBuf.empty(cfg.L, N, cfg.H, cfg.cap, cfg.Dh, tdt, pool=True)
    sdev.fill_kv(cfg, pool.kv, torch.from_numpy(lens0).cuda(), 0, False)
    tok0, _, _ = synth.tokens_host(cfg, lens0, 0, False)
    pool.tokens.copy_(torch.from_numpy(tok0))
    pool.len.copy_(torch.from_numpy(lens0))
    ng = (N + G - 1) // G
    rect = sd.SeqBuf.empty(cfg.L, N, cfg.H, cfg.cap, cfg.Dh, tdt, groups=ng)
    logits = torch.empty((N, cfg.D1, cfg.V), dtype=sdev.TORCH_DT[cfg.logit_dtype], device="cuda")
    kv_new = torch.empty((cfg.L, 2, N, cfg.H, cfg.D1, cfg.Dh), dtype=tdt, device="cuda")
    ws = sd.workspace(N, cfg.D)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    check_rounds = {0, 1, R // 2, R - 1}
    lcheck = 0
    hist = []
    for r in range(R):
        say("exspec round", r)
        plant, miss, draft = synth.plan_greedy(cfg, r)
        keep = sdev.fill_logits(cfg, r, plant, logits)
        sdev.fill_kvnew(cfg, r, kv_new)
        if r == R - 1:
            rect.kv.view(torch.uint8).fill_(CANARY_KV)  # every layer of the last gather is checked
            rect.tokens.fill_(CANARY_I32)
        elif r in check_rounds:
            rect.kv[lcheck].view(torch.uint8).fill_(CANARY_KV)
            rect.tokens.fill_(CANARY_I32)
        order, uni, wid, nu = sd.group_by_len(pool.len, G)
        sd.gather(pool, rect, order, G, uni, status=status)
        dd = torch.from_numpy(draft).cuda()
        acc, nxt = sd.verify_greedy(logits, dd, ws=ws, status=status)
        sd.append(pool, kv_new, dd, acc, nxt, status=status)
        rec = dict(order=order.cpu().numpy(), uni=uni.cpu().numpy(), wid=wid.cpu().numpy(), nu=int(nu.item()),
                   acc=acc.cpu().numpy(), nxt=nxt.cpu().numpy())
        if r in check_rounds:
            rec["rkv"] = to_np_raw(rect.kv[lcheck])
            rec["rtok"] = rect.tokens.cpu().numpy()
            rec["rpos"] = rect.pos.cpu().numpy()
            rec["rmask"] = rect.mask.cpu().numpy()
            rec["rwidth"] = rect.width.cpu().numpy()
        hist.append(rec)
        del keep
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    final_kv = {l: to_np_raw(pool.kv[l]) for l in (0, cfg.L - 1)}
    final_tok, final_len = pool.tokens.cpu().numpy(), pool.len.cpu().numpy()

    say("exspec oracle")
    lens = lens0.copy()
    tok = tok0.copy()
    kvs = {l: synth.kv_host(cfg, lens0, 0, False, layer0=l, nlayers=1) for l in (0, cfg.L - 1)}
    rounds = []
    for r in range(R):
        h = hist[r]
        order, uni, wid, nu = oracle.group_by_len(lens, G)
        if r == R - 1:
            last_gather = dict(order=order, uni=uni, wid=wid, lens=lens.copy(), tok=tok.copy())
        assert np.array_equal(h["order"], order) and np.array_equal(h["uni"], uni), "round %d grouping" % r
        assert np.array_equal(h["wid"], wid) and h["nu"] == nu
        if r == 0:
            assert nu == ng, "the first round's batches are all same-length"
        if r in check_rounds:
            want = oracle.gather(kvs[lcheck], tok, lens, order, G, uni, cfg.cap)
            for g in range(ng):
                sl = slice(g * G, g * G + G)
                if uni[g]:
                    assert np.all(h["rkv"][:, sl].view(np.uint8) == CANARY_KV), "uniform batch was copied"
                    continue
                W = wid[g]
                assert h["rwidth"][g] == W
                assert bytes_equal(h["rkv"][:, sl, :, :W], want["kv"][0, :, sl, :, :W]), "round %d group %d" % (r, g)
                for name in ("tokens", "pos", "mask"):
                    assert np.array_equal(h["r" + {"tokens": "tok", "pos": "pos", "mask": "mask"}[name]][sl, :W],
                                          want[name][sl, :W]), name
        plant, miss, draft = synth.plan_greedy(cfg, r)
        lg = synth.logits_host(cfg, r, plant)
        oacc, onxt, _ = oracle.verify_greedy(lg, draft, N, cfg.D, cfg.V)
        assert np.array_equal(h["acc"], oacc) and np.array_equal(h["nxt"], onxt), "round %d verify" % r
        rounds.append((draft, oacc, onxt))
        for l in kvs:
            kvn = synth.kvnew_host(cfg, r, layer0=l, nlayers=1)
            lens_l = lens.copy()
            tok_l = tok.copy() if l == 0 else None
            oracle.append(kvs[l], tok_l, lens_l, np.arange(N), kvn, draft, oacc, onxt)
            if l == 0:
                new_tok, new_lens = tok_l, lens_l
        tok, lens = new_tok, new_lens
    assert np.array_equal(final_len, lens)
    assert np.array_equal(final_tok, tok)
    for l in kvs:
        assert bytes_equal(final_kv[l], kvs[l][0]), "final pool layer %d" % l

    # every layer: the last round's gather and the final pool, each layer's pool
    # regenerated and carried through the rounds' appends by the oracle (its
    # OpenMP build: a layer of the pool is 1.1 GB)
    lg_ = last_gather
    with oracle.threaded():
        for l in range(cfg.L):
            say("exspec every layer", l)
            kv_l = synth.kv_host(cfg, lens0, 0, False, layer0=l, nlayers=1)
            lens_l = lens0.copy()
            for r in range(R):
                if r == R - 1:
                    want = oracle.gather(kv_l, lg_["tok"], lens_l, lg_["order"], G, lg_["uni"], cfg.cap)
                    for g in range(ng):
                        sl = slice(g * G, g * G + G)
                        if lg_["uni"][g]:
                            assert bool((rect.kv[l][:, sl].view(torch.uint8) == CANARY_KV).all()), \
                                "layer %d: uniform batch %d was copied" % (l, g)
                            continue
                        W = int(lg_["wid"][g])
                        assert device_equal(rect.kv[l][:, sl, :, :W], want["kv"][0, :, sl, :, :W]), \
                            "last gather, layer %d group %d" % (l, g)
                    del want
                draft, oacc, onxt = rounds[r]
                kvn = synth.kvnew_host(cfg, r, layer0=l, nlayers=1)
                oracle.append(kv_l, None, lens_l, np.arange(N), kvn, draft, oacc, onxt)
            assert np.array_equal(lens_l, final_len)
            assert device_equal(pool.kv[l], kv_l[0]), "final pool layer %d" % l
            del kv_l
