"""GPU parity of the paged KV cache (block tables; the realignment as metadata)
against the oracle: admit, append, gather and retire leave the pages, block
table, free stack, token ids and lengths byte for byte as the oracle's paged
functions do (one fixed allocation policy on both sides), and over chained
rounds of the generated workloads the gathered rectangle equals the EQSPEC
oracle's.  Status bits leave every buffer unchanged."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sdev
from tests.full_layers import check_chain_final_layers
from tests.gpu_util import bytes_equal, from_np_raw, say, to_np_raw

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_kv_realignment_amd as m
    return m


def _dev_state(sd, st, tdt):
    """The oracle's paged state copied to the device."""
    return sd.PagedKV(from_np_raw(st.pages, tdt), torch.from_numpy(st.bt).cuda(), torch.from_numpy(st.free).cuda(),
                      torch.from_numpy(st.n_free).cuda(), torch.from_numpy(st.tokens).cuda(),
                      torch.from_numpy(st.len).cuda())


def _same_state(cache, st, what):
    torch.cuda.synchronize()
    assert bytes_equal(to_np_raw(cache.pages), st.pages), what + ": pages"
    assert np.array_equal(cache.block_table.cpu().numpy(), st.bt), what + ": block table"
    nf = int(st.n_free[0])
    assert int(cache.n_free.item()) == nf, what + ": n_free"
    assert np.array_equal(cache.free_pages.cpu().numpy()[:nf], st.free[:nf]), what + ": free stack"
    assert np.array_equal(cache.len.cpu().numpy(), st.len), what + ": len"
    assert np.array_equal(cache.tokens.cpu().numpy(), st.tokens), what + ": tokens"


def _rect(rng, B, L, H, Dh, dt_np, lens, S, cap):
    kv = np.zeros((L, 2, B, H, cap, Dh), dt_np)
    tok = np.zeros((B, cap), np.int32)
    for b in range(B):
        pad = S - lens[b]
        kv[:, :, b, :, pad:S] = rng.standard_normal((L, 2, H, lens[b], Dh))
        tok[b, pad:S] = rng.integers(1, 500, lens[b])
    return kv, tok


def _seqbuf(sd, kv, tok, lens, S, tdt):
    B, cap = tok.shape
    return sd.SeqBuf(from_np_raw(kv, tdt), torch.from_numpy(tok).cuda(),
                     torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda(),
                     torch.zeros((B, cap), dtype=torch.int32, device="cuda"),
                     torch.zeros((B, cap), dtype=torch.int8, device="cuda"),
                     torch.tensor([S], dtype=torch.int32, device="cuda"))


# (numpy dtype, torch dtype, head_dim): 16-byte units per position 1, 4, 8, 16, 256
_GEOMS = [(np.float32, torch.float32, 4), (np.float16, torch.float16, 32), (np.float16, torch.float16, 64),
          (np.float16, torch.float16, 128), (np.float32, torch.float32, 1024)]


@pytest.mark.parametrize("seed", range(10))
def test_paged_random(sd, seed):
    """Random geometry, page sizes 1-64, a shuffled free stack, a batch of pool
    rows that is not the whole pool: admit, rounds of append (with the
    rectangle view), gather, retire and readmit, each compared with the oracle."""
    rng = np.random.default_rng(1100 + seed)
    dt_np, tdt, Dh = _GEOMS[seed % len(_GEOMS)]
    page = int([1, 3, 16, 64, 7][seed % 5])
    rows = int(rng.integers(2, 10))
    B = int(rng.integers(1, rows + 1))
    D = int(rng.integers(0, 6)) if seed % 3 else 0
    L, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    maxlen = 40 if Dh == 1024 else int(rng.integers(10, 300))
    rounds = 3
    cap = maxlen + rounds * (D + 1)
    mb = -(-cap // page)
    n_pages = rows * mb + int(rng.integers(0, 5))
    say("paged random", seed, rows, B, D, L, H, Dh, page, n_pages)
    st = oracle.PagedState(L, H, Dh, n_pages, page, mb, rows, dt_np,
                           free_order=rng.permutation(n_pages).astype(np.int32))
    cache = _dev_state(sd, st, tdt)
    prow = rng.permutation(rows)[:B].astype(np.int32)
    lens = rng.integers(0, maxlen, B).astype(np.int32)
    S = int(lens.max())
    kv, tok = _rect(rng, B, L, H, Dh, dt_np, lens, S, cap)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    prow_d = torch.from_numpy(prow).cuda()
    sd.paged_admit(cache, _seqbuf(sd, kv, tok, lens, S, tdt), rows=prow_d, status=status)
    oracle.paged_admit(st, kv, tok, lens, S, rows=prow)
    _same_state(cache, st, "admit")
    for r in range(rounds):
        kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(dt_np)
        acc = rng.integers(0, D + 1, B).astype(np.int32)
        draft = rng.integers(1, 500, (B, D)).astype(np.int32)
        nxt = rng.integers(1, 500, B).astype(np.int32)
        rt = torch.full((B, cap), -7, dtype=torch.int32, device="cuda")
        rp = torch.full((B, cap), -7, dtype=torch.int32, device="cuda")
        rm = torch.full((B, cap), 7, dtype=torch.int8, device="cuda")
        width = torch.zeros(1, dtype=torch.int32, device="cuda")
        sd.paged_append(cache, from_np_raw(kv_new, tdt), torch.from_numpy(draft).cuda(), torch.from_numpy(acc).cuda(),
                        torch.from_numpy(nxt).cuda(), rows=prow_d, pad_token=int(seed % 3), width=width,
                        rect_tokens=rt, rect_pos=rp, rect_mask=rm, status=status)
        view = oracle.paged_append(st, kv_new, draft, acc, nxt, rows=prow, pad_token=int(seed % 3), rect_cap=cap)
        _same_state(cache, st, "append round %d" % r)
        W = view["width"]
        assert int(width.item()) == W
        for got, want, canary in ((rt, view["tokens"], -7), (rp, view["pos"], -7), (rm, view["mask"], 7)):
            g = got.cpu().numpy()
            assert np.array_equal(g[:, :W], want) and np.all(g[:, W:] == canary)
    out = sd.SeqBuf.empty(L, B, H, cap, Dh, tdt)
    sd.paged_gather(cache, out, rows=prow_d, status=status)
    want = oracle.paged_gather(st, rows=prow, cap_out=cap)
    torch.cuda.synchronize()
    W = want["width"]
    assert int(out.width[0].item()) == W
    assert bytes_equal(to_np_raw(out.kv)[..., :W, :], want["kv"])
    for k in ("tokens", "pos", "mask"):
        assert np.array_equal(getattr(out, k).cpu().numpy()[:, :W], want[k]), k
    assert np.array_equal(out.len.cpu().numpy(), want["len"])
    # retire half of the batch, then admit fresh content into those rows
    gone = prow[: max(1, B // 2)]
    sd.paged_retire(cache, torch.from_numpy(gone).cuda(), status=status)
    oracle.paged_retire(st, gone)
    _same_state(cache, st, "retire")
    lens2 = rng.integers(0, maxlen, gone.size).astype(np.int32)
    S2 = int(lens2.max())
    kv2, tok2 = _rect(rng, gone.size, L, H, Dh, dt_np, lens2, S2, cap)
    sd.paged_admit(cache, _seqbuf(sd, kv2, tok2, lens2, S2, tdt), rows=torch.from_numpy(gone).cuda(), status=status)
    oracle.paged_admit(st, kv2, tok2, lens2, S2, rows=gone)
    _same_state(cache, st, "readmit")
    assert int(status.item()) == 0


def _run_chain_paged(sd, name, rounds, check_rounds, layers):
    """`rounds` chained greedy verify + paged append rounds, checked round by
    round against the oracle's EQSPEC chain on the contiguous rectangle."""
    cfg = synth.CONFIGS[name]
    say("paged chain", name, "setup")
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    w = sdev.GreedyRounds(cfg, rounds)
    page = 16
    mb = -(-cfg.cap // page)
    rect = sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, tdt)
    w.load_initial(rect)
    cache = sd.PagedKV.empty(cfg.L, cfg.B, cfg.H, cfg.Dh, cfg.B * mb, page, mb, tdt)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sd.paged_admit(cache, rect, status=status)
    ws = sd.workspace(cfg.B, cfg.D)
    width = torch.zeros(1, dtype=torch.int32, device="cuda")
    rt = torch.zeros((cfg.B, cfg.cap), dtype=torch.int32, device="cuda")
    rp = torch.zeros_like(rt)
    rm = torch.zeros((cfg.B, cfg.cap), dtype=torch.int8, device="cuda")
    hist = {k: [] for k in ("acc", "nxt", "tokens", "pos", "mask", "len", "width")}
    kv_hist = {}
    for r in range(rounds):
        say("paged chain", name, "round", r)
        acc, nxt = sd.verify_greedy(w.logits[r], w.drafts[r], ws=ws, status=status)
        sd.paged_append(cache, w.kv_new[r], w.drafts[r], acc, nxt, width=width, rect_tokens=rt, rect_pos=rp,
                        rect_mask=rm, status=status)
        hist["acc"].append(acc.clone())
        hist["nxt"].append(nxt.clone())
        for k, t in (("tokens", rt), ("pos", rp), ("mask", rm), ("len", cache.len), ("width", width)):
            hist[k].append(t.clone())
        if r in check_rounds:
            sd.paged_gather(cache, rect, status=status)
            kv_hist[r] = {l: to_np_raw(rect.kv[l]) for l in layers}
            kv_hist[r]["width"] = int(rect.width[0].item())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    hist = {k: [t.cpu().numpy() for t in v] for k, v in hist.items()}

    say("paged chain", name, "oracle")
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
                assert kv_hist[r]["width"] == Wr
                assert bytes_equal(kv_hist[r][l][..., :Wr, :], out["kv"][0, ..., :Wr, :]), \
                    "round %d layer %d KV" % (r, l)
        Wr = out["width"]
        assert int(hist["width"][r][0]) == Wr
        assert np.array_equal(hist["len"][r], out["len"])
        for k in ("tokens", "pos", "mask"):
            assert np.array_equal(hist[k][r][:, :Wr], out[k][:, :Wr]), "round %d %s" % (r, k)
        state, lens, S, tok, mask = new_state, out["len"], Wr, out["tokens"], out["mask"]
    # every layer of the final paged cache, through a gather into the rectangle
    say("paged chain", name, "final gather")
    rect.kv.view(torch.uint8).fill_(0xA5)
    sd.paged_gather(cache, rect, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(rect.width[0].item()) == S
    Wf = check_chain_final_layers(cfg, w.lens0, w.width0, oacc_hist, lambda l: rect.kv[l], "paged chain " + name,
                                  canary=0xA5)
    assert Wf == S


def test_paged_chain_7b_mha(sd):
    cfg = synth.CONFIGS["7b-mha"]
    _run_chain_paged(sd, "7b-mha", cfg.rounds, {0, cfg.rounds // 2, cfg.rounds - 1}, [0, cfg.L - 1])


def test_paged_chain_8b_gqa(sd):
    cfg = synth.CONFIGS["8b-gqa"]
    _run_chain_paged(sd, "8b-gqa", cfg.rounds, {0, cfg.rounds // 2, cfg.rounds - 1}, [0, cfg.L // 2, cfg.L - 1])


def test_paged_status_bits_write_nothing(sd):
    """Too few free pages, a row past its block capacity, a rectangle view too
    narrow, accepted lengths out of range, a bad row, duplicate rows, a free
    stack whose top is no page id or whose count exceeds the pages, and an
    admit into a row that is not empty: each sets its bit and changes nothing
    (duplicates: the bit only; the result is undefined)."""
    rng = np.random.default_rng(1200)
    L, H, Dh, page, B, D = 1, 2, 8, 4, 3, 3

    def state(lens):
        st = oracle.PagedState(L, H, Dh, 8, page, 3, 4, np.float16, free_order=rng.permutation(8).astype(np.int32))
        kv, tok = _rect(rng, B, L, H, Dh, np.float16, lens, 12, 12)
        oracle.paged_admit(st, kv, tok, lens, 12)
        return st, kv, tok

    base, kv, tok = state(np.array([4, 7, 2], np.int32))     # 1 + 2 + 1 pages held, 4 free
    long_row, _, _ = state(np.array([4, 10, 2], np.int32))   # row 1 holds 10 of its 12 positions
    short = base.copy()
    short.n_free[0] = 2                                      # 2 free; acc 3 everywhere needs 3
    bad_page = base.copy()
    bad_page.free[bad_page.n_free[0] - 1] = 999              # the top of the free stack is no page
    bad_count = base.copy()
    bad_count.n_free[0] = 99                                 # more free entries than pages
    kv_new = torch.from_numpy(rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float16)).cuda()
    draft = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")

    def I(*v):
        return torch.tensor(v, dtype=torch.int32, device="cuda")

    cases = [("pages", short, I(3, 3, 3), None, 16, sd.S_CAPACITY),
             ("row capacity", long_row, I(0, 3, 0), None, 16, sd.S_CAPACITY),
             ("rect too narrow", base, I(3, 3, 3), None, 8, sd.S_CAPACITY),
             ("accept range", base, I(0, 4, 0), None, 16, sd.S_LEN_RANGE),
             ("accept negative", base, I(0, -1, 0), None, 16, sd.S_LEN_RANGE),
             ("bad row", base, I(0, 0, 0), I(0, 1, 9), 16, sd.S_LEN_RANGE),
             ("dup rows", base, I(0, 0, 0), I(0, 1, 1), 16, sd.S_ROWS_DUP),
             ("free page id", bad_page, I(3, 3, 3), None, 16, sd.S_LEN_RANGE),
             ("free count", bad_count, I(3, 3, 3), None, 16, sd.S_LEN_RANGE)]
    for what, st, acc, rows, rcap, bit in cases:
        say("paged status", what)
        cache = _dev_state(sd, st, torch.float16)
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        rt = torch.full((B, rcap), -7, dtype=torch.int32, device="cuda")
        sd.paged_append(cache, kv_new, draft, acc, nxt, rows=rows, rect_tokens=rt, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) & bit, what
        if bit != sd.S_ROWS_DUP:
            _same_state(cache, st, what)
            assert np.all(rt.cpu().numpy() == -7), what
    say("paged status", "admit into a row that is not empty")
    cache = _dev_state(sd, base, torch.float16)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sd.paged_admit(cache, _seqbuf(sd, kv[:, :, :1], tok[:1], np.array([4], np.int32), 12, torch.float16), rows=I(1),
                   status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & sd.S_LEN_RANGE
    _same_state(cache, base, "admit into a row that is not empty")


def test_paged_host_errors(sd):
    say("paged host errors")
    cache = sd.PagedKV.empty(1, 2, 1, 8, 4, 4, 2, torch.float16)
    kv_new = torch.zeros((1, 2, 2, 1, 3, 8), dtype=torch.float16, device="cuda")
    z = torch.zeros(2, dtype=torch.int32, device="cuda")
    dr = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(sd.SpecDecError) as e:  # the committed KV inside the page pool
        sd.paged_append(cache, cache.pages.view(-1)[:kv_new.numel()].view(kv_new.shape), dr, z, z)
    assert e.value.code == -4
    with pytest.raises(sd.SpecDecError) as e:  # 8-byte positions
        c4 = sd.PagedKV.empty(1, 2, 1, 4, 4, 4, 2, torch.float16)
        sd.paged_append(c4, torch.zeros((1, 2, 2, 1, 3, 4), dtype=torch.float16, device="cuda"), dr, z, z)
    assert e.value.code == -5
    out = sd.SeqBuf.empty(1, 3, 1, 8, 8, torch.float16)
    with pytest.raises(ValueError):  # one pool row per rectangle row
        sd.paged_gather(cache, out, rows=z)
    with pytest.raises(sd.SpecDecError) as e:  # a rectangle of another head count
        sd.paged_gather(cache, sd.SeqBuf.empty(1, 2, 2, 8, 8, torch.float16))
    assert e.value.code == -1


def test_paged_largest_batch(sd):
    """B = 1024 batch entries (the limit) over a pool of 1100 rows with pages of
    4 positions: two rounds of append, then gather, against the oracle."""
    rng = np.random.default_rng(1210)
    rows, B, D, L, H, Dh, page = 1100, 1024, 3, 1, 1, 8, 4
    maxlen = 30
    cap = maxlen + 2 * (D + 1)
    mb = -(-cap // page)
    n_pages = rows * mb
    say("paged largest batch", rows, B)
    st = oracle.PagedState(L, H, Dh, n_pages, page, mb, rows, np.float16,
                           free_order=rng.permutation(n_pages).astype(np.int32))
    cache = _dev_state(sd, st, torch.float16)
    prow = rng.permutation(rows)[:B].astype(np.int32)
    lens = rng.integers(0, maxlen, B).astype(np.int32)
    S = int(lens.max())
    kv, tok = _rect(rng, B, L, H, Dh, np.float16, lens, S, cap)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    prow_d = torch.from_numpy(prow).cuda()
    sd.paged_admit(cache, _seqbuf(sd, kv, tok, lens, S, torch.float16), rows=prow_d, status=status)
    oracle.paged_admit(st, kv, tok, lens, S, rows=prow)
    for r in range(2):
        kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float16)
        acc = rng.integers(0, D + 1, B).astype(np.int32)
        draft = rng.integers(1, 500, (B, D)).astype(np.int32)
        nxt = rng.integers(1, 500, B).astype(np.int32)
        rt = torch.full((B, cap), -7, dtype=torch.int32, device="cuda")
        sd.paged_append(cache, torch.from_numpy(kv_new).cuda(), torch.from_numpy(draft).cuda(),
                        torch.from_numpy(acc).cuda(), torch.from_numpy(nxt).cuda(), rows=prow_d, rect_tokens=rt,
                        status=status)
        view = oracle.paged_append(st, kv_new, draft, acc, nxt, rows=prow, rect_cap=cap)
        _same_state(cache, st, "largest batch round %d" % r)
        assert np.array_equal(rt.cpu().numpy()[:, :view["width"]], view["tokens"])
    out = sd.SeqBuf.empty(L, B, H, cap, Dh, torch.float16)
    sd.paged_gather(cache, out, rows=prow_d, status=status)
    want = oracle.paged_gather(st, rows=prow, cap_out=cap)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert bytes_equal(to_np_raw(out.kv)[..., :want["width"], :], want["kv"])


def test_paged_append_many_passes(sd):
    """An append whose speculative KV holds more 16-byte units (4.2M) than the
    copy grid takes in one pass (3,072 workgroups of 1,024 units), so each copy
    workgroup loops; no row map, pages of 16; against the oracle."""
    rng = np.random.default_rng(1220)
    rows, B, D, L, H, Dh, page = 128, 128, 7, 4, 32, 128, 16
    maxlen = 12
    cap = maxlen + D + 1
    mb = -(-cap // page)
    n_pages = rows * mb
    say("paged many passes", L, B, H, D + 1, Dh)
    st = oracle.PagedState(L, H, Dh, n_pages, page, mb, rows, np.float16,
                           free_order=rng.permutation(n_pages).astype(np.int32))
    cache = _dev_state(sd, st, torch.float16)
    lens = rng.integers(0, maxlen, B).astype(np.int32)
    S = int(lens.max())
    kv, tok = _rect(rng, B, L, H, Dh, np.float16, lens, S, cap)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sd.paged_admit(cache, _seqbuf(sd, kv, tok, lens, S, torch.float16), status=status)
    oracle.paged_admit(st, kv, tok, lens, S)
    kv_new = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float16)
    assert kv_new.size * 2 // 16 > 3072 * 1024
    acc = rng.integers(0, D + 1, B).astype(np.int32)
    draft = rng.integers(1, 500, (B, D)).astype(np.int32)
    nxt = rng.integers(1, 500, B).astype(np.int32)
    sd.paged_append(cache, torch.from_numpy(kv_new).cuda(), torch.from_numpy(draft).cuda(),
                    torch.from_numpy(acc).cuda(), torch.from_numpy(nxt).cuda(), status=status)
    oracle.paged_append(st, kv_new, draft, acc, nxt)
    _same_state(cache, st, "many passes")
    assert int(status.item()) == 0
