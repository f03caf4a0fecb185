"""GPU parity of realignment: EQSPEC chains of the generated workloads and
edge cases, bit-exact against the oracle, with canaries on what must not be
written; status bits forced from the host."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sdev
from oracle import brute
from tests import invariants as inv
from tests.full_layers import check_chain_final_layers, device_equal
from tests.gpu_util import bytes_equal, from_np_raw, say, to_np_raw

pytestmark = pytest.mark.gpu

CANARY_KV = 0xA5
CANARY_I32 = -7
CANARY_I8 = 7


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_kv_realignment_amd as m
    return m


def _poison(buf):
    buf.kv.view(torch.uint8).fill_(CANARY_KV)
    buf.tokens.fill_(CANARY_I32)
    buf.pos.fill_(CANARY_I32)
    buf.mask.fill_(CANARY_I8)
    buf.len.fill_(CANARY_I32)
    buf.width.fill_(CANARY_I32)


def _device_rect(sd, host_kv, tok, pos, mask, lens, width, tdt):
    L, _, B, H, cap, Dh = host_kv.shape
    buf = sd.SeqBuf(from_np_raw(host_kv, tdt), torch.from_numpy(tok).cuda(),
                    torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda(), torch.from_numpy(pos).cuda(),
                    torch.from_numpy(mask).cuda(), torch.tensor([width], dtype=torch.int32, device="cuda"))
    return buf


@pytest.mark.parametrize("seed", range(8))
def test_eqspec_random_small(sd, seed):
    """Random rectangles (ragged lengths, zero-length rows, D = 0, several element
    sizes) against the oracle and the per-sequence brute force."""
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 20))
    D = int(rng.integers(0, 7))
    L, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    dt_np, tdt, Dh = [(np.float32, torch.float32, 4), (np.float16, torch.float16, 8), (np.float16, torch.float16, 64),
                      (np.float32, torch.float32, 32)][seed % 4]
    cap = int(rng.integers(D + 2, 90))
    lens = rng.integers(0, cap - D, B).astype(np.int32)
    S = int(lens.max())
    say("eqspec random", seed, B, D, L, H, Dh, cap)
    kv = np.zeros((L, 2, B, H, cap, Dh), dt_np)
    tok = np.zeros((B, cap), np.int32)
    pos = np.zeros((B, cap), np.int32)
    mask = np.zeros((B, cap), np.int8)
    for b in range(B):
        pad = S - lens[b]
        kv[:, :, b, :, pad:S] = rng.standard_normal((L, 2, H, lens[b], Dh))
        tok[b, pad:S] = rng.integers(1, 500, lens[b])
        mask[b, pad:S] = 1
        pos[b, pad:S] = np.arange(lens[b])
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(dt_np)
    acc = rng.integers(0, D + 1, B).astype(np.int32)
    draft = rng.integers(1, 500, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 500, B).astype(np.int32)
    cap_out = S + D + 1 + int(rng.integers(0, 5))

    src = _device_rect(sd, kv, tok, pos, mask, lens, S, tdt)
    dst = sd.SeqBuf.empty(L, B, H, cap_out, Dh, tdt)
    _poison(dst)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sd.realign_eqspec(src, dst, from_np_raw(kv_new, tdt), torch.from_numpy(draft).cuda(),
                      torch.from_numpy(acc).cuda(), torch.from_numpy(nxt).cuda(), pad_token=0, status=status)
    torch.cuda.synchronize()
    want = oracle.realign_eqspec(kv, kv_new, lens, S, tok, mask, acc, nxt, draft, cap_out=cap_out)
    W = want["width"]
    assert int(status.item()) == 0
    assert int(dst.width.item()) == W
    assert np.array_equal(dst.len.cpu().numpy(), want["len"])
    for name in ("tokens", "pos", "mask"):
        got = getattr(dst, name).cpu().numpy()
        assert np.array_equal(got[:, :W], want[name][:, :W]), name
        assert np.all(got[:, W:] == (CANARY_I8 if name == "mask" else CANARY_I32)), name + " written past width"
    gkv = to_np_raw(dst.kv)
    assert bytes_equal(gkv[..., :W, :], want["kv"][..., :W, :])
    assert np.all(gkv[..., W:, :].view(np.uint8) == CANARY_KV), "KV written past width"
    committed = [list(draft[b, :acc[b]]) + [int(nxt[b])] for b in range(B)]
    inv.check_round(tok, mask, S, dst.tokens.cpu().numpy(), dst.pos.cpu().numpy(), dst.mask.cpu().numpy(),
                    want["len"], W, acc, committed, D)


def test_eqspec_tiny_equals_unbatched(sd):
    """Tiny workload: one greedy verify + one realign on the GPU equals the
    unbatched per-sequence brute force run of each row."""
    cfg = synth.CONFIGS["tiny"]
    say("eqspec tiny")
    w = sdev.GreedyRounds(cfg, 1)
    src = sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, torch.float32)
    dst = sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, torch.float32)
    w.load_initial(src)
    _poison(dst)
    acc, nxt = sd.verify_greedy(w.logits[0], w.drafts[0])
    sd.realign_eqspec(src, dst, w.kv_new[0], w.drafts[0], acc, nxt)
    torch.cuda.synchronize()
    lens, S = w.lens0, w.width0
    kv0 = synth.kv_host(cfg, lens, S, True)
    kvn = synth.kvnew_host(cfg, 0)
    assert bytes_equal(to_np_raw(src.kv), kv0)
    logits = synth.logits_host(cfg, 0, w.plans[0][0])
    W = int(dst.width.item())
    gk = to_np_raw(dst.kv)
    for b in range(cfg.B):
        a, committed = brute.greedy_one(logits[b * cfg.D1:(b + 1) * cfg.D1], w.plans[0][2][b])
        assert (a, committed[-1]) == (acc[b].item(), nxt[b].item())
        t1, k1 = brute.advance(list(w.tok0[b, S - lens[b]:S]), kv0[:, :, b, :, S - lens[b]:S], committed, kvn[:, :, b])
        c1 = len(t1)
        assert int(dst.len[b].item()) == c1
        assert list(dst.tokens[b, W - c1:W].cpu().numpy()) == t1
        assert list(dst.pos[b, W - c1:W].cpu().numpy()) == list(range(c1))
        assert bytes_equal(gk[:, :, b, :, W - c1:W], k1)
        assert np.all(gk[:, :, b, :, :W - c1] == 0)


def _run_chain(sd, name, rounds, check_rounds, layers):
    """`rounds` chained greedy verify + EQSPEC rounds on the GPU, checked round by
    round against the oracle run on the same generated inputs.  Token ids,
    position ids, mask, lengths, widths, accepted lengths and next tokens are
    compared at every round; KV bytes of `layers` at `check_rounds`, and of every
    layer after the last round."""
    cfg = synth.CONFIGS[name]
    say("chain", name, "setup")
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    w = sdev.GreedyRounds(cfg, rounds)
    bufs = [sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, tdt) for _ in range(2)]
    w.load_initial(bufs[0])
    ws = sd.workspace(cfg.B, cfg.D)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    hist = {k: [] for k in ("acc", "nxt", "tokens", "pos", "mask", "len", "width")}
    kv_hist = {}
    for r in range(rounds):
        src, dst = bufs[r % 2], bufs[(r + 1) % 2]
        _poison(dst)
        say("chain", name, "round", r)
        acc, nxt = sd.verify_greedy(w.logits[r], w.drafts[r], ws=ws, status=status)
        sd.realign_eqspec(src, dst, w.kv_new[r], w.drafts[r], acc, nxt, status=status)
        hist["acc"].append(acc.clone())
        hist["nxt"].append(nxt.clone())
        for k in ("tokens", "pos", "mask", "len", "width"):
            hist[k].append(getattr(dst, k).clone())
        if r in check_rounds:
            kv_hist[r] = {l: to_np_raw(dst.kv[l]) for l in layers}
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    hist = {k: [t.cpu().numpy() for t in v] for k, v in hist.items()}

    say("chain", name, "oracle")
    lens, S = w.lens0.copy(), w.width0
    tok, mask = w.tok0.copy(), w.mask0.copy()
    state = {l: synth.kv_host(cfg, lens, S, True, layer0=l, nlayers=1) for l in layers}
    oacc_hist = []
    for r in range(rounds):
        plant, miss, draft = w.plans[r]
        logits = synth.logits_host(cfg, r, plant)
        oacc, onxt, _ = oracle.verify_greedy(logits, draft, cfg.B, cfg.D, cfg.V)
        oacc_hist.append(oacc)
        assert np.array_equal(hist["acc"][r], oacc), "round %d accept_len" % r
        assert np.array_equal(hist["nxt"][r], onxt), "round %d next_token" % r
        new_state = {}
        out = None
        for l in layers:
            kvn = synth.kvnew_host(cfg, r, layer0=l, nlayers=1)
            out = oracle.realign_eqspec(state[l], kvn, lens, S, tok, mask, oacc, onxt, draft)
            new_state[l] = out["kv"]
            if r in check_rounds:
                Wr = out["width"]
                g = kv_hist[r][l]
                assert bytes_equal(g[..., :Wr, :], out["kv"][0, ..., :Wr, :]), "round %d layer %d KV" % (r, l)
                assert np.all(g[..., Wr:, :].view(np.uint8) == CANARY_KV), "round %d layer %d past width" % (r, l)
        Wr = out["width"]
        assert int(hist["width"][r][0]) == Wr
        assert np.array_equal(hist["len"][r], out["len"])
        for k in ("tokens", "pos", "mask"):
            assert np.array_equal(hist[k][r][:, :Wr], out[k][:, :Wr]), "round %d %s" % (r, k)
            assert np.all(hist[k][r][:, Wr:] == (CANARY_I8 if k == "mask" else CANARY_I32))
        committed = [list(draft[b, :oacc[b]]) + [int(onxt[b])] for b in range(cfg.B)]
        inv.check_round(tok, mask, S, out["tokens"], out["pos"], out["mask"], out["len"], Wr, oacc, committed, cfg.D)
        state, lens, S, tok, mask = new_state, out["len"], Wr, out["tokens"], out["mask"]
    final = bufs[rounds % 2]
    Wf = check_chain_final_layers(cfg, w.lens0, w.width0, oacc_hist, lambda l: final.kv[l], "eqspec chain " + name,
                                  canary=CANARY_KV)
    assert Wf == S


def test_eqspec_chain_7b_mha(sd):
    cfg = synth.CONFIGS["7b-mha"]
    _run_chain(sd, "7b-mha", cfg.rounds, {0, 1, cfg.rounds // 2, cfg.rounds - 1}, [0, cfg.L - 1])


def test_eqspec_chain_8b_gqa(sd):
    cfg = synth.CONFIGS["8b-gqa"]
    _run_chain(sd, "8b-gqa", cfg.rounds, {0, 1, cfg.rounds // 2, cfg.rounds - 1}, [0, cfg.L // 2, cfg.L - 1])


def test_eqspec_status_bits_write_nothing(sd):
    """Device-detected conditions: capacity too small, accepted length out of
    range, a length above the width.  Each sets its bit and writes nothing."""
    rng = np.random.default_rng(77)
    B, D, L, H, Dh, cap = 4, 3, 1, 2, 8, 20
    lens = np.array([5, 9, 0, 7], np.int32)
    S = 9
    kv = rng.standard_normal((L, 2, B, H, cap, Dh)).astype(np.float16)
    tok = np.zeros((B, cap), np.int32)
    pos = np.zeros((B, cap), np.int32)
    mask = np.zeros((B, cap), np.int8)
    for b in range(B):
        mask[b, S - lens[b]:S] = 1
    kv_new = torch.from_numpy(rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float16)).cuda()
    draft = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    cases = [("capacity", np.array([3, 3, 0, 0], np.int32), S + 3, None, sd.S_CAPACITY),
             ("accept range", np.array([0, 4, 0, 0], np.int32), cap, None, sd.S_LEN_RANGE),
             ("accept negative", np.array([0, -1, 0, 0], np.int32), cap, None, sd.S_LEN_RANGE),
             ("len above width", np.array([0, 0, 0, 0], np.int32), cap, np.array([5, 10, 0, 7], np.int32),
              sd.S_LEN_RANGE)]
    for what, acc, cap_out, bad_lens, bit in cases:
        say("eqspec status", what)
        src = _device_rect(sd, kv, tok, pos, mask, lens if bad_lens is None else bad_lens, S, torch.float16)
        dst = sd.SeqBuf.empty(L, B, H, cap_out, Dh, torch.float16)
        _poison(dst)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        sd.realign_eqspec(src, dst, kv_new, draft, torch.from_numpy(acc).cuda(), nxt, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) & bit, what
        assert np.all(to_np_raw(dst.kv).view(np.uint8) == CANARY_KV), what
        assert np.all(dst.tokens.cpu().numpy() == CANARY_I32) and np.all(dst.len.cpu().numpy() == CANARY_I32)


def test_eqspec_host_errors(sd):
    say("eqspec host errors")
    B, D, L, H, Dh, cap = 2, 2, 1, 1, 8, 16
    a = sd.SeqBuf.empty(L, B, H, cap, Dh, torch.float16)
    kv_new = torch.zeros((L, 2, B, H, D + 1, Dh), dtype=torch.float16, device="cuda")
    z = torch.zeros(B, dtype=torch.int32, device="cuda")
    dr = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    with pytest.raises(sd.SpecDecError) as e:
        sd.realign_eqspec(a, a, kv_new, dr, z, z)
    assert e.value.code == -4  # in and out overlap
    odd = sd.SeqBuf.empty(L, B, H, cap, 4, torch.float16)  # 8-byte positions
    with pytest.raises(sd.SpecDecError) as e:
        sd.realign_eqspec(odd, sd.SeqBuf.empty(L, B, H, cap, 4, torch.float16),
                          torch.zeros((L, 2, B, H, D + 1, 4), dtype=torch.float16, device="cuda"), dr, z, z)
    assert e.value.code == -5


# ------------------------------------------------------------------ stochastic workload

def test_stochastic_round_realign(sd):
    """Sampled verify then EQSPEC realign of the fp16 32x32x128 cache (B=32, D=8)."""
    cfg = synth.CONFIGS["stoch"]
    say("stoch setup")
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    lens = synth.lengths(cfg)
    S = int(lens.max())
    p, q, draft, u_acc, u_draw = synth.sampled_round(cfg, 0)
    src = sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, tdt)
    dst = sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, tdt)
    sdev.fill_kv(cfg, src.kv, torch.from_numpy(lens).cuda(), S, True)
    tok, pos, mask = synth.tokens_host(cfg, lens, S, True)
    src.tokens.copy_(torch.from_numpy(tok))
    src.pos.copy_(torch.from_numpy(pos))
    src.mask.copy_(torch.from_numpy(mask))
    src.len.copy_(torch.from_numpy(lens))
    src.width.fill_(S)
    kv_new = torch.empty((cfg.L, 2, cfg.B, cfg.H, cfg.D1, cfg.Dh), dtype=tdt, device="cuda")
    sdev.fill_kvnew(cfg, 0, kv_new)
    _poison(dst)
    say("stoch run")
    dev_draft = torch.from_numpy(draft).cuda()
    acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in (p, q)), dev_draft,
                                torch.from_numpy(u_acc).cuda(), torch.from_numpy(u_draw).cuda())
    sd.realign_eqspec(src, dst, kv_new, dev_draft, acc, nxt)
    torch.cuda.synchronize()
    gacc, gnxt = acc.cpu().numpy(), nxt.cpu().numpy()
    oacc, onxt, _ = oracle.verify_sample(p, q, draft, u_acc, u_draw)
    assert np.array_equal(gacc, oacc)
    ambiguous = np.nonzero(gnxt != onxt)[0]
    assert len(ambiguous) == 0, "a draw fell inside the tie band; see the band rule"
    W = None
    with oracle.threaded():  # every layer (1 GB each): the OpenMP build of the same oracle
        for l in range(cfg.L):
            say("stoch oracle, layer", l)
            kv_l = synth.kv_host(cfg, lens, S, True, layer0=l, nlayers=1)
            kvn_l = synth.kvnew_host(cfg, 0, layer0=l, nlayers=1)
            out = oracle.realign_eqspec(kv_l, kvn_l, lens, S, tok, mask, oacc, onxt, draft)
            W = out["width"]
            assert device_equal(dst.kv[l][..., :W, :], out["kv"][0, ..., :W, :]), "layer %d" % l
            assert bool((dst.kv[l][..., W:, :].contiguous().view(torch.uint8) == CANARY_KV).all())
            if l == 0:
                meta = {k: out[k] for k in ("tokens", "pos", "mask", "len")}
            del kv_l, out
    assert int(dst.width.item()) == W
    assert np.array_equal(dst.len.cpu().numpy(), meta["len"])
    for k in ("tokens", "pos", "mask"):
        assert np.array_equal(getattr(dst, k).cpu().numpy()[:, :W], meta[k][:, :W]), k


@pytest.mark.parametrize("shape", [
    # B, D, L, H, Dh, dtype, cap: the largest batch, the widest position, an odd number of 16-byte units
    (1024, 3, 1, 1, 8, np.float16, 14),
    (3, 2, 1, 1, 1024, np.float32, 10),
    (5, 4, 2, 3, 96, np.float16, 40),
    (7, 0, 1, 2, 8, np.float32, 9),
])
def test_eqspec_limits(sd, shape):
    B, D, L, H, Dh, dt_np, cap = shape
    tdt = torch.float16 if dt_np == np.float16 else torch.float32
    rng = np.random.default_rng(B + Dh)
    lens = rng.integers(0, cap - D - 1, B).astype(np.int32)
    S = int(lens.max())
    say("eqspec limits", shape)
    kv = np.zeros((L, 2, B, H, cap, Dh), dt_np)
    tok = np.zeros((B, cap), np.int32)
    pos = np.zeros((B, cap), np.int32)
    mask = np.zeros((B, cap), np.int8)
    for b in range(B):
        pad = S - lens[b]
        kv[:, :, b, :, pad:S] = rng.standard_normal((L, 2, H, lens[b], Dh))
        tok[b, pad:S] = rng.integers(1, 99, lens[b])
        mask[b, pad:S] = 1
        pos[b, pad:S] = np.arange(lens[b])
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(dt_np)
    acc = rng.integers(0, D + 1, B).astype(np.int32)
    draft = rng.integers(1, 99, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 99, B).astype(np.int32)
    src = _device_rect(sd, kv, tok, pos, mask, lens, S, tdt)
    dst = sd.SeqBuf.empty(L, B, H, cap, Dh, tdt)
    _poison(dst)
    sd.realign_eqspec(src, dst, from_np_raw(kv_new, tdt), torch.from_numpy(draft).cuda(), torch.from_numpy(acc).cuda(),
                      torch.from_numpy(nxt).cuda())
    torch.cuda.synchronize()
    want = oracle.realign_eqspec(kv, kv_new, lens, S, tok, mask, acc, nxt, draft, cap_out=cap)
    W = want["width"]
    assert int(dst.width.item()) == W
    gkv = to_np_raw(dst.kv)
    assert bytes_equal(gkv[..., :W, :], want["kv"][..., :W, :])
    assert np.all(gkv[..., W:, :].view(np.uint8) == CANARY_KV)
    for name in ("tokens", "pos", "mask"):
        assert np.array_equal(getattr(dst, name).cpu().numpy()[:, :W], want[name][:, :W]), name
