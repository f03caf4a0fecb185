"""GPU parity of the in-place EQSPEC realignment: the rectangle after the call
equals the oracle's out-of-place EQSPEC result on [0, S'), bit for bit, and
positions [S', cap) keep the bytes they held.  Covers moves to lower and to
higher positions over many chunks, rows wider than one chunk of token ids,
every 16-byte unit count per position from 1 to 256, chained rounds of the
generated workloads, status bits and host errors."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sdev
from tests import invariants as inv
from tests.full_layers import check_chain_final_layers
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


def _rect(rng, B, L, H, Dh, dt_np, lens, S, cap):
    """Left-padded rectangle of width S in buffers of capacity cap: zero KV on
    pad, canaries on [S, cap) and on pad token ids, position ids and mask."""
    kv = np.zeros((L, 2, B, H, cap, Dh), dt_np)
    kv[..., S:, :].view(np.uint8)[...] = CANARY_KV
    tok = np.full((B, cap), CANARY_I32, np.int32)
    pos = np.full((B, cap), CANARY_I32, np.int32)
    mask = np.full((B, cap), CANARY_I8, np.int8)
    for b in range(B):
        pad = S - lens[b]
        kv[:, :, b, :, pad:S] = rng.standard_normal((L, 2, H, lens[b], Dh))
        tok[b, pad:S] = rng.integers(1, 500, lens[b])
        mask[b, :S] = 0
        mask[b, pad:S] = 1
        pos[b, :S] = 0
        pos[b, pad:S] = np.arange(lens[b])
    return kv, tok, pos, mask


def _check_inplace(sd, kv, tok, pos, mask, lens, S, kv_new, acc, draft, nxt, tdt, pad_token=0, zero_pad=False):
    """Runs the in-place realignment on the device copy of the rectangle and
    compares it with the oracle and with the input bytes past the new width."""
    B = lens.shape[0]
    buf = sd.SeqBuf(from_np_raw(kv, tdt), torch.from_numpy(tok).cuda(),
                    torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda(), torch.from_numpy(pos).cuda(),
                    torch.from_numpy(mask).cuda(), torch.tensor([S], dtype=torch.int32, device="cuda"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sd.realign_eqspec_inplace(buf, from_np_raw(kv_new, tdt), torch.from_numpy(draft).cuda(),
                              torch.from_numpy(acc).cuda(), torch.from_numpy(nxt).cuda(), pad_token=pad_token,
                              status=status, zero_pad=zero_pad)
    torch.cuda.synchronize()
    want = oracle.realign_eqspec(kv, kv_new, lens, S, tok, mask, acc, nxt, draft, pad_token=pad_token)
    W = want["width"]
    assert int(status.item()) == 0
    assert int(buf.width.item()) == W
    assert np.array_equal(buf.len.cpu().numpy(), want["len"])
    for name, before in (("tokens", tok), ("pos", pos), ("mask", mask)):
        got = getattr(buf, name).cpu().numpy()
        assert np.array_equal(got[:, :W], want[name][:, :W]), name
        assert np.array_equal(got[:, W:], before[:, W:]), name + " changed past the new width"
    gkv = to_np_raw(buf.kv)
    assert bytes_equal(gkv[..., :W, :], want["kv"][..., :W, :])
    assert bytes_equal(gkv[..., W:, :], kv[..., W:, :]), "KV changed past the new width"
    committed = [list(draft[b, :acc[b]]) + [int(nxt[b])] for b in range(B)]
    inv.check_round(tok, mask, S, buf.tokens.cpu().numpy(), buf.pos.cpu().numpy(), buf.mask.cpu().numpy(),
                    want["len"], W, acc, committed, draft.shape[1], pad_token=pad_token)
    return W


# (dtype, torch dtype, head_dim): 16-byte units per position 1, 4, 8, 16, 256
_GEOMS = [(np.float32, torch.float32, 4), (np.float16, torch.float16, 32), (np.float16, torch.float16, 64),
          (np.float16, torch.float16, 128), (np.float32, torch.float32, 1024)]


@pytest.mark.parametrize("seed", range(12))
def test_inplace_random(sd, seed):
    """Random rectangles: ragged lengths with zero-length rows, D = 0, widths
    above the longest row (moves to lower positions by more than a chunk), and
    rows long enough for many chunks in either direction."""
    rng = np.random.default_rng(900 + seed)
    dt_np, tdt, Dh = _GEOMS[seed % len(_GEOMS)]
    U = Dh * np.dtype(dt_np).itemsize // 16
    B = int(rng.integers(1, 12))
    D = int(rng.integers(0, 7)) if seed % 3 else 0
    L, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    maxlen = 60 if U == 256 else int(rng.integers(20, 700))
    lens = rng.integers(0, maxlen, B).astype(np.int32)
    if seed % 4 == 1:
        lens[rng.integers(0, B)] = 0
    S = int(lens.max()) + (int(rng.integers(0, 200)) if seed % 2 else 0)
    cap = S + D + 1 + int(rng.integers(0, 4))
    say("inplace random", seed, B, D, L, H, Dh, S, cap)
    kv, tok, pos, mask = _rect(rng, B, L, H, Dh, dt_np, lens, S, cap)
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(dt_np)
    acc = rng.integers(0, D + 1, B).astype(np.int32)
    draft = rng.integers(1, 500, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 500, B).astype(np.int32)
    _check_inplace(sd, kv, tok, pos, mask, lens, S, kv_new, acc, draft, nxt, tdt, pad_token=int(seed % 3))


@pytest.mark.parametrize("shape", [
    # B, D, L, H, Dh, dtype, cap: the largest batch (one row per thread of the
    # prologue), the widest position, an odd number of 16-byte units, no drafts
    (1024, 3, 1, 2, 8, np.float16, 14),
    (3, 2, 1, 1, 1024, np.float32, 10),
    (5, 4, 2, 3, 96, np.float16, 40),
    (7, 0, 1, 2, 8, np.float32, 9),
])
def test_inplace_limits(sd, shape):
    B, D, L, H, Dh, dt_np, cap = shape
    tdt = torch.float16 if dt_np == np.float16 else torch.float32
    rng = np.random.default_rng(7 * B + Dh)
    lens = rng.integers(0, cap - D - 1, B).astype(np.int32)
    S = int(lens.max())
    say("inplace limits", shape)
    kv, tok, pos, mask = _rect(rng, B, L, H, Dh, dt_np, lens, S, cap)
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(dt_np)
    acc = rng.integers(0, D + 1, B).astype(np.int32)
    draft = rng.integers(1, 500, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 500, B).astype(np.int32)
    _check_inplace(sd, kv, tok, pos, mask, lens, S, kv_new, acc, draft, nxt, tdt)


def test_inplace_long_token_rows(sd):
    """Rows of several chunks of token ids (a chunk is 4 ids per thread of a
    1024-thread workgroup), both move directions."""
    rng = np.random.default_rng(31)
    B, D, L, H, Dh = 6, 5, 1, 1, 4
    lens = np.array([9000, 1, 8200, 0, 4500, 8999], np.int32)
    acc = np.array([5, 0, 2, 5, 1, 0], np.int32)  # rows 0 and 5 move down, the others up
    S = int(lens.max())
    cap = S + D + 1
    say("inplace long token rows")
    kv, tok, pos, mask = _rect(rng, B, L, H, Dh, np.float32, lens, S, cap)
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float32)
    draft = rng.integers(1, 500, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 500, B).astype(np.int32)
    _check_inplace(sd, kv, tok, pos, mask, lens, S, kv_new, acc, draft, nxt, torch.float32)


def test_inplace_uniform_full_accept(sd):
    """Every row of one length accepting everything: no row moves (append only)."""
    rng = np.random.default_rng(32)
    B, D, L, H, Dh = 5, 4, 2, 2, 64
    lens = np.full(B, 300, np.int32)
    acc = np.full(B, D, np.int32)
    S = 300
    say("inplace uniform")
    kv, tok, pos, mask = _rect(rng, B, L, H, Dh, np.float16, lens, S, S + D + 1)
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float16)
    draft = rng.integers(1, 500, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 500, B).astype(np.int32)
    _check_inplace(sd, kv, tok, pos, mask, lens, S, kv_new, acc, draft, nxt, torch.float16)


def _run_chain_inplace(sd, name, rounds, check_rounds, layers):
    """`rounds` chained greedy verify + in-place EQSPEC rounds on one rectangle,
    checked round by round against the oracle's out-of-place realignment."""
    cfg = synth.CONFIGS[name]
    say("inplace chain", name, "setup")
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    w = sdev.GreedyRounds(cfg, rounds)
    buf = sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, tdt)
    w.load_initial(buf)
    ws = sd.workspace(cfg.B, cfg.D)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    hist = {k: [] for k in ("acc", "nxt", "tokens", "pos", "mask", "len", "width")}
    kv_hist = {}
    for r in range(rounds):
        say("inplace chain", name, "round", r)
        acc, nxt = sd.verify_greedy(w.logits[r], w.drafts[r], ws=ws, status=status)
        sd.realign_eqspec_inplace(buf, w.kv_new[r], w.drafts[r], acc, nxt, status=status)
        hist["acc"].append(acc.clone())
        hist["nxt"].append(nxt.clone())
        for k in ("tokens", "pos", "mask", "len", "width"):
            hist[k].append(getattr(buf, k).clone())
        if r in check_rounds:
            kv_hist[r] = {l: to_np_raw(buf.kv[l]) for l in layers}
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    hist = {k: [t.cpu().numpy() for t in v] for k, v in hist.items()}

    say("inplace chain", name, "oracle")
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
        new_state, out = {}, None
        for l in layers:
            kvn = synth.kvnew_host(cfg, r, layer0=l, nlayers=1)
            out = oracle.realign_eqspec(state[l], kvn, lens, S, tok, mask, oacc, onxt, draft)
            new_state[l] = out["kv"]
            if r in check_rounds:
                Wr = out["width"]
                assert bytes_equal(kv_hist[r][l][..., :Wr, :], out["kv"][0, ..., :Wr, :]), \
                    "round %d layer %d KV" % (r, l)
        Wr = out["width"]
        assert int(hist["width"][r][0]) == Wr
        assert np.array_equal(hist["len"][r], out["len"])
        for k in ("tokens", "pos", "mask"):
            assert np.array_equal(hist[k][r][:, :Wr], out[k][:, :Wr]), "round %d %s" % (r, k)
        state, lens, S, tok, mask = new_state, out["len"], Wr, out["tokens"], out["mask"]
    Wf = check_chain_final_layers(cfg, w.lens0, w.width0, oacc_hist, lambda l: buf.kv[l], "inplace chain " + name)
    assert Wf == S


def test_inplace_chain_7b_mha(sd):
    cfg = synth.CONFIGS["7b-mha"]
    _run_chain_inplace(sd, "7b-mha", cfg.rounds, {0, 1, cfg.rounds // 2, cfg.rounds - 1}, [0, cfg.L - 1])


def test_inplace_chain_8b_gqa(sd):
    cfg = synth.CONFIGS["8b-gqa"]
    _run_chain_inplace(sd, "8b-gqa", cfg.rounds, {0, 1, cfg.rounds // 2, cfg.rounds - 1},
                       [0, cfg.L // 2, cfg.L - 1])


@pytest.mark.parametrize("seed", range(8))
def test_inplace_zero_pad_garbage_input_pad(sd, seed):
    """An input whose pad positions hold arbitrary bytes (as a left-padded
    prefill leaves them): the zero-pad mode gives the EQSPEC result on [0, S')
    byte for byte, rows that move either way and rows that only append alike;
    positions past the new width keep their bytes."""
    rng = np.random.default_rng(1300 + seed)
    dt_np, tdt, Dh = _GEOMS[seed % len(_GEOMS)]
    U = Dh * np.dtype(dt_np).itemsize // 16
    B = int(rng.integers(2, 12))
    D = int(rng.integers(0, 6))
    L, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    maxlen = 60 if U == 256 else int(rng.integers(20, 700))
    lens = rng.integers(0, maxlen, B).astype(np.int32)
    lens[0] = 0 if seed % 2 else lens[0]
    S = int(lens.max()) + (int(rng.integers(0, 100)) if seed % 3 == 0 else 0)
    cap = S + D + 1 + int(rng.integers(0, 4))
    say("inplace zero pad", seed, B, D, L, H, Dh, S, cap)
    kv, tok, pos, mask = _rect(rng, B, L, H, Dh, dt_np, lens, S, cap)
    raw = kv.view(np.uint8)
    for b in range(B):   # garbage bytes on every row's pad, all layers, K and V, heads
        nb = (S - lens[b]) * Dh * np.dtype(dt_np).itemsize
        if nb:
            raw[:, :, b, :, :nb] = rng.integers(0, 256, raw[:, :, b, :, :nb].shape, dtype=np.uint8)
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(dt_np)
    acc = rng.integers(0, D + 1, B).astype(np.int32)
    draft = rng.integers(1, 500, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 500, B).astype(np.int32)
    _check_inplace(sd, kv, tok, pos, mask, lens, S, kv_new, acc, draft, nxt, tdt, zero_pad=True)


def test_inplace_default_mode_keeps_garbage_pad(sd):
    """The default in-place mode leaves bytes below both the old and the new pad
    untouched: the precondition (a zero input pad) is real, and the zero-pad
    mode is the one for such inputs."""
    rng = np.random.default_rng(1400)
    B, D, L, H, Dh = 3, 2, 1, 1, 8
    lens = np.array([4, 9, 6], np.int32)
    S, cap = 9, 14
    kv, tok, pos, mask = _rect(rng, B, L, H, Dh, np.float16, lens, S, cap)
    kv[:, :, 0, :, :S - lens[0]] = 7.0            # row 0: pad 5, new pad >= 5 - 3
    buf = sd.SeqBuf(from_np_raw(kv, torch.float16), torch.from_numpy(tok).cuda(),
                    torch.from_numpy(lens).cuda(), torch.from_numpy(pos).cuda(), torch.from_numpy(mask).cuda(),
                    torch.tensor([S], dtype=torch.int32, device="cuda"))
    kv_new = torch.zeros((L, 2, B, H, D + 1, Dh), dtype=torch.float16, device="cuda")
    acc = torch.tensor([0, 2, 1], dtype=torch.int32, device="cuda")  # S' = 12; row 0's new pad is 7
    z = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    sd.realign_eqspec_inplace(buf, kv_new, z, acc, torch.ones(B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert bool((buf.kv[0, :, 0, :, :5].float() == 7.0).all()), "positions [0, 5) of row 0 were rewritten"


def test_inplace_status_bits_write_nothing(sd):
    """Capacity too small for the new width, accepted length out of range, a
    length above the width: each sets its bit and leaves every buffer as it was."""
    rng = np.random.default_rng(78)
    B, D, L, H, Dh = 4, 3, 1, 2, 8
    lens = np.array([5, 9, 0, 7], np.int32)
    S, cap = 9, 12
    kv, tok, pos, mask = _rect(rng, B, L, H, Dh, np.float16, lens, S, cap)
    kv_new = torch.from_numpy(rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float16)).cuda()
    draft = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    cases = [("capacity", np.array([0, 3, 0, 0], np.int32), lens, sd.S_CAPACITY),
             ("accept range", np.array([0, 4, 0, 0], np.int32), lens, sd.S_LEN_RANGE),
             ("accept negative", np.array([0, -1, 0, 0], np.int32), lens, sd.S_LEN_RANGE),
             ("len above width", np.array([0, 0, 0, 0], np.int32), np.array([5, 10, 0, 7], np.int32),
              sd.S_LEN_RANGE)]
    for what, acc, ln, bit in cases:
        say("inplace status", what)
        buf = sd.SeqBuf(from_np_raw(kv, torch.float16), torch.from_numpy(tok).cuda(), torch.from_numpy(ln).cuda(),
                        torch.from_numpy(pos).cuda(), torch.from_numpy(mask).cuda(),
                        torch.tensor([S], dtype=torch.int32, device="cuda"))
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        sd.realign_eqspec_inplace(buf, kv_new, draft, torch.from_numpy(acc).cuda(), nxt, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) & bit, what
        assert bytes_equal(to_np_raw(buf.kv), kv), what
        assert np.array_equal(buf.tokens.cpu().numpy(), tok) and np.array_equal(buf.pos.cpu().numpy(), pos)
        assert np.array_equal(buf.mask.cpu().numpy(), mask) and np.array_equal(buf.len.cpu().numpy(), ln)
        assert int(buf.width.item()) == S


def test_inplace_host_errors(sd):
    say("inplace host errors")
    B, D, L, H, Dh, cap = 2, 2, 1, 1, 8, 16
    a = sd.SeqBuf.empty(L, B, H, cap, Dh, torch.float16)
    b = sd.SeqBuf.empty(L, B, H, cap, Dh, torch.float16)
    kv_new = torch.zeros((L, 2, B, H, D + 1, Dh), dtype=torch.float16, device="cuda")
    z = torch.zeros(B, dtype=torch.int32, device="cuda")
    dr = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    with pytest.raises(sd.SpecDecError) as e:  # two different rectangles
        sd.specdec_realign_kv(sd.EQSPEC_INPLACE, a, b, None, B, 0, None, kv_new, dr, z, z)
    assert e.value.code == -1
    with pytest.raises(sd.SpecDecError) as e:  # the committed KV inside the cache
        sd.realign_eqspec_inplace(a, a.kv.view(-1)[:kv_new.numel()].view(kv_new.shape), dr, z, z)
    assert e.value.code == -4
    with pytest.raises(sd.SpecDecError) as e:  # accepted lengths stored over the row lengths
        sd.realign_eqspec_inplace(a, kv_new, dr, a.len, z)
    assert e.value.code == -4
    with pytest.raises(sd.SpecDecError) as e:  # 8-byte positions
        o = sd.SeqBuf.empty(L, B, H, cap, 4, torch.float16)
        sd.realign_eqspec_inplace(o, torch.zeros((L, 2, B, H, D + 1, 4), dtype=torch.float16, device="cuda"),
                                  dr, z, z)
    assert e.value.code == -5
