"""GPU parity of greedy verification fused into the paged append: one call that
leaves per-workgroup keys and lets the append kernel finish verification gives,
byte for byte, what specdec_verify_greedy followed by specdec_paged_append
gives (those separate calls are checked against the oracle elsewhere), on
random inputs with ties, drafts out of range, zero-length rows and D = 0."""
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


def _rect(sd, rng, B, L, H, Dh, tdt, lens, S, cap):
    kv = np.zeros((L, 2, B, H, cap, Dh), np.float32)
    tok = np.zeros((B, cap), np.int32)
    pos = np.zeros((B, cap), np.int32)
    mask = np.zeros((B, cap), np.int8)
    for b in range(B):
        pad = S - lens[b]
        kv[:, :, b, :, pad:S] = rng.standard_normal((L, 2, H, lens[b], Dh))
        tok[b, pad:S] = rng.integers(1, 500, lens[b])
        mask[b, pad:S] = 1
        pos[b, pad:S] = np.arange(lens[b])
    mk = lambda: sd.SeqBuf(torch.from_numpy(kv).to("cuda", tdt), torch.from_numpy(tok).cuda(),
                           torch.from_numpy(lens).cuda(), torch.from_numpy(pos).cuda(), torch.from_numpy(mask).cuda(),
                           torch.tensor([S], dtype=torch.int32, device="cuda"))
    return mk(), mk()


def _logits(rng, B, D, V, ldt, draft_bad=False):
    logits = np.round(rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)  # many ties
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    am = logits.argmax(-1)
    for b in range(B):
        k = int(rng.integers(0, D + 1))
        draft[b, :k] = am[b, :k]
    if draft_bad and D > 0:
        draft[0, -1] = V + 3
    return torch.from_numpy(logits).to("cuda", ldt), torch.from_numpy(draft).cuda()


@pytest.mark.parametrize("seed", range(6))
def test_fused_paged_random(sd, seed):
    rng = np.random.default_rng(1700 + seed)
    ldt = [torch.float32, torch.bfloat16][seed % 2]
    B = int(rng.integers(1, 30))
    D = int(rng.integers(0, 7)) if seed % 3 else 0
    V = int(rng.integers(100, 20000))
    L, H, Dh, page = 2, 2, 64, int([1, 16, 5][seed % 3])
    lens = rng.integers(0, 200, B).astype(np.int32)
    S = int(lens.max())
    cap = S + 3 * (D + 1)
    mb = -(-cap // page)
    say("fused paged", seed, B, D, V, page)
    rect, _ = _rect(sd, rng, B, L, H, Dh, torch.float16, lens, S, cap)
    perm = torch.from_numpy(rng.permutation(B * mb + 3).astype(np.int32))
    ca = sd.PagedKV.empty(L, B, H, Dh, B * mb + 3, page, mb, torch.float16, free_order=perm)
    cb = sd.PagedKV.empty(L, B, H, Dh, B * mb + 3, page, mb, torch.float16, free_order=perm)
    sd.paged_admit(ca, rect)
    sd.paged_admit(cb, rect)
    for r in range(3):
        logits, draft = _logits(rng, B, D, V, ldt)
        kv_new = torch.from_numpy(rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float16)).cuda()
        views = [(torch.full((B, cap), -7, dtype=torch.int32, device="cuda"),
                  torch.full((B, cap), -7, dtype=torch.int32, device="cuda"),
                  torch.full((B, cap), 7, dtype=torch.int8, device="cuda"),
                  torch.zeros(1, dtype=torch.int32, device="cuda")) for _ in range(2)]
        acc1, nxt1 = sd.verify_greedy(logits, draft)
        sd.paged_append(ca, kv_new, draft, acc1, nxt1, width=views[0][3], rect_tokens=views[0][0],
                        rect_pos=views[0][1], rect_mask=views[0][2])
        acc2, nxt2 = sd.verify_paged_append(logits, draft, cb, kv_new, width=views[1][3], rect_tokens=views[1][0],
                                            rect_pos=views[1][1], rect_mask=views[1][2])
        torch.cuda.synchronize()
        assert torch.equal(acc1, acc2) and torch.equal(nxt1, nxt2), r
        for x, y in zip(*views):
            assert torch.equal(x, y), r
        for k in ("block_table", "free_pages", "n_free", "tokens", "len"):
            assert torch.equal(getattr(ca, k), getattr(cb, k)), (r, k)
        assert bytes_equal(to_np_raw(ca.pages), to_np_raw(cb.pages)), r


def test_fused_host_errors(sd):
    say("fused host errors")
    B, D, V = 3, 2, 100
    logits = torch.zeros((B, D + 1, V), device="cuda")
    draft = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    kv_new = torch.zeros((1, 2, B, 1, D + 1, 8), dtype=torch.float16, device="cuda")
    cache = sd.PagedKV.empty(1, B, 1, 8, 16, 4, 4, torch.float16)
    with pytest.raises(sd.SpecDecError) as e:  # workspace too small
        sd.verify_paged_append(logits, draft, cache, kv_new, ws=torch.empty(8, dtype=torch.uint8, device="cuda"))
    assert e.value.code == -3
    big = torch.zeros((700, 4, 10), device="cuda")  # B * (D+1) above 2048
    with pytest.raises(sd.SpecDecError) as e:
        sd.verify_paged_append(big, torch.zeros((700, 3), dtype=torch.int32, device="cuda"),
                               sd.PagedKV.empty(1, 700, 1, 8, 2800, 4, 4, torch.float16),
                               torch.zeros((1, 2, 700, 1, 4, 8), dtype=torch.float16, device="cuda"))
    assert e.value.code == -1
