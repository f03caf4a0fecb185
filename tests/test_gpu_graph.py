"""Chained rounds captured in one HIP graph (greedy verification + paged
append; greedy verification + in-place realignment): every replay, with the
program's own eager work (a reset of the cache) and synchronisations between
replays, reproduces the eager rounds byte for byte."""
import numpy as np
import pytest
import torch

from tests.gpu_util import bytes_equal, say, to_np_raw

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_kv_realignment_amd as m
    return m


def test_paged_rounds_graph_replays(sd):
    rng = np.random.default_rng(1800)
    B, D, V, L, H, Dh, page, R = 12, 4, 5000, 2, 2, 64, 8, 10
    lens = rng.integers(20, 300, B).astype(np.int32)
    S = int(lens.max())
    cap = S + R * (D + 1)
    mb = -(-cap // page)
    say("graph replay", B, D, V, R)
    kv = np.zeros((L, 2, B, H, cap, Dh), np.float16)
    tok = np.zeros((B, cap), np.int32)
    for b in range(B):
        kv[:, :, b, :, S - lens[b]:S] = rng.standard_normal((L, 2, H, lens[b], Dh))
        tok[b, S - lens[b]:S] = rng.integers(1, V, lens[b])
    rect = sd.SeqBuf(torch.from_numpy(kv).cuda(), torch.from_numpy(tok).cuda(), torch.from_numpy(lens).cuda(),
                     torch.zeros((B, cap), dtype=torch.int32, device="cuda"),
                     torch.zeros((B, cap), dtype=torch.int8, device="cuda"),
                     torch.tensor([S], dtype=torch.int32, device="cuda"))
    cache = sd.PagedKV.empty(L, B, H, Dh, B * mb, page, mb, torch.float16)
    logits = torch.from_numpy(rng.standard_normal((R, B, D + 1, V)).astype(np.float32)).cuda()
    drafts = rng.integers(0, V, (R, B, D)).astype(np.int32)
    am = logits.argmax(-1).cpu().numpy()
    for r in range(R):
        for b in range(B):
            k = int(rng.integers(0, D + 1))
            drafts[r, b, :k] = am[r, b, :k]
    drafts = torch.from_numpy(drafts).cuda()
    kv_new = torch.from_numpy(rng.standard_normal((R, L, 2, B, H, D + 1, Dh)).astype(np.float16)).cuda()
    ws = sd.workspace(B, D)
    acc = torch.zeros((R, B), dtype=torch.int32, device="cuda")
    nxt = torch.zeros((R, B), dtype=torch.int32, device="cuda")
    width = torch.zeros(1, dtype=torch.int32, device="cuda")
    view = (torch.zeros((B, cap), dtype=torch.int32, device="cuda"),
            torch.zeros((B, cap), dtype=torch.int32, device="cuda"),
            torch.zeros((B, cap), dtype=torch.int8, device="cuda"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    sd.paged_admit(cache, rect, status=status)
    torch.cuda.synchronize()
    names = ("pages", "block_table", "free_pages", "n_free", "tokens", "len", "sync")
    initial = {k: getattr(cache, k).clone() for k in names}

    def reset():  # eager work between replays: the cache back to its state after the admission
        for k in names:
            getattr(cache, k).copy_(initial[k])
        torch.cuda.synchronize()

    def rounds():
        for r in range(R):
            sd.verify_greedy(logits[r], drafts[r], ws=ws, status=status, accept_len=acc[r], next_token=nxt[r])
            sd.paged_append(cache, kv_new[r], drafts[r], acc[r], nxt[r], width=width, rect_tokens=view[0],
                            rect_pos=view[1], rect_mask=view[2], status=status)

    def snapshot():
        torch.cuda.synchronize()
        return ([t.clone() for t in (acc, nxt, width, *view, cache.block_table, cache.n_free, cache.tokens,
                                      cache.len)], to_np_raw(cache.pages), cache.free_pages[:int(cache.n_free.item())]
                .clone())

    reset()
    rounds()
    want = snapshot()
    assert int(status.item()) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rounds()
    for rep in range(3):
        reset()
        acc.zero_()
        nxt.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for i, (x, y) in enumerate(zip(got[0], want[0])):
            assert torch.equal(x, y), (rep, i)
        assert bytes_equal(got[1], want[1]), rep
        assert torch.equal(got[2], want[2]), rep
    assert int(status.item()) == 0


def test_inplace_rounds_graph_replays(sd):
    """Chained rounds of greedy verification + in-place EQSPEC realignment of a
    left-padded rectangle captured in one HIP graph: every replay, with an
    eager reset of the rectangle and synchronisations between replays,
    reproduces the eager rounds byte for byte (accepted lengths, next tokens,
    KV, token ids, position ids, mask, lengths and width)."""
    rng = np.random.default_rng(1900)
    B, D, V, L, H, Dh, R = 12, 4, 5000, 2, 2, 64, 10
    lens = rng.integers(20, 300, B).astype(np.int32)
    S = int(lens.max())
    cap = S + R * (D + 1)
    say("graph replay in place", B, D, V, R)
    kv = np.zeros((L, 2, B, H, cap, Dh), np.float16)
    tok = np.zeros((B, cap), np.int32)
    pos = np.zeros((B, cap), np.int32)
    mask = np.zeros((B, cap), np.int8)
    for b in range(B):
        kv[:, :, b, :, S - lens[b]:S] = rng.standard_normal((L, 2, H, lens[b], Dh))
        tok[b, S - lens[b]:S] = rng.integers(1, V, lens[b])
        pos[b, S - lens[b]:S] = np.arange(lens[b])
        mask[b, S - lens[b]:S] = 1
    buf = sd.SeqBuf(torch.from_numpy(kv).cuda(), torch.from_numpy(tok).cuda(), torch.from_numpy(lens).cuda(),
                    torch.from_numpy(pos).cuda(), torch.from_numpy(mask).cuda(),
                    torch.tensor([S], dtype=torch.int32, device="cuda"))
    logits = torch.from_numpy(rng.standard_normal((R, B, D + 1, V)).astype(np.float32)).cuda()
    drafts = rng.integers(0, V, (R, B, D)).astype(np.int32)
    am = logits.argmax(-1).cpu().numpy()
    for r in range(R):
        for b in range(B):
            k = int(rng.integers(0, D + 1))
            drafts[r, b, :k] = am[r, b, :k]
    drafts = torch.from_numpy(drafts).cuda()
    kv_new = torch.from_numpy(rng.standard_normal((R, L, 2, B, H, D + 1, Dh)).astype(np.float16)).cuda()
    ws = sd.workspace(B, D)
    acc = torch.zeros((R, B), dtype=torch.int32, device="cuda")
    nxt = torch.zeros((R, B), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    names = ("kv", "tokens", "pos", "mask", "len", "width")
    initial = {k: getattr(buf, k).clone() for k in names}

    def reset():  # eager work between replays: the rectangle back to its first state
        for k in names:
            getattr(buf, k).copy_(initial[k])
        torch.cuda.synchronize()

    def rounds():
        for r in range(R):
            sd.verify_greedy(logits[r], drafts[r], ws=ws, status=status, accept_len=acc[r], next_token=nxt[r])
            sd.realign_eqspec_inplace(buf, kv_new[r], drafts[r], acc[r], nxt[r], status=status)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (acc, nxt, buf.tokens, buf.pos, buf.mask, buf.len, buf.width)], to_np_raw(buf.kv)

    reset()
    rounds()
    want = snapshot()
    assert int(status.item()) == 0 and int(want[0][0].sum()) > 0  # some drafts were accepted
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rounds()
    for rep in range(3):
        reset()
        acc.zero_()
        nxt.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for i, (x, y) in enumerate(zip(got[0], want[0])):
            assert torch.equal(x, y), (rep, i)
        assert bytes_equal(got[1], want[1]), rep
    assert int(status.item()) == 0


def test_sample_logits_graph_replays(sd):
    """Sampled verification from logits with a top-p nucleus, three calls
    captured in one HIP graph: every replay gives the eager accepted lengths,
    next tokens and nucleus thresholds (the workspace holds nothing between
    calls, so no clearing is captured)."""
    rng = np.random.default_rng(2000)
    B, D, V, R = 6, 3, 9000, 3
    say("graph replay sampled from logits", B, D, V, R)
    tl = torch.from_numpy((rng.standard_normal((R, B, D + 1, V)) * 2).astype(np.float32)).cuda()
    dl = (tl[:, :, :D] + torch.from_numpy((rng.standard_normal((R, B, D, V)) * 0.5).astype(np.float32)).cuda())
    dl = dl.contiguous()
    draft = dl.argmax(-1).to(torch.int32).contiguous()
    u_acc = torch.from_numpy(rng.random((R, B, D)).astype(np.float32)).cuda()
    u_draw = torch.from_numpy(rng.random((R, B, D + 1)).astype(np.float32)).cuda()
    ws = sd.sample_workspace(B, D, V)
    acc = torch.zeros((R, B), dtype=torch.int32, device="cuda")
    nxt = torch.zeros((R, B), dtype=torch.int32, device="cuda")
    cut = torch.zeros((R, B * (2 * D + 1)), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def calls():
        for r in range(R):
            sd.verify_sample_logits(tl[r], dl[r], draft[r], u_acc[r], u_draw[r], 0.8, top_p=0.9, ws=ws,
                                    status=status, accept_len=acc[r], next_token=nxt[r], cutoff=cut[r])

    calls()
    torch.cuda.synchronize()
    want = [t.clone() for t in (acc, nxt, cut)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        for t in (acc, nxt, cut):
            t.zero_()
        ws.fill_(0x5A)  # eager work between replays that disturbs the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip((acc, nxt, cut), want)):
            assert torch.equal(x, y), (rep, i)
    assert int(status.item()) == 0
