"""GPU parity of sampled verification from logits (temperature softmax and the
top-p nucleus fused into the kernels) against the oracle.  Both sides decide in
fp64 from the same logits; they differ only in the rounding of exp and of the
order of sums (and, for the nucleus, in summing masses as 2^-41 fixed-point
integers), so a decision may differ only where the oracle's own values put it
within the band (1e-6 relative) of its threshold, and the GPU's outcome must
then be one of the admissible ones.  A nucleus threshold the GPU chose within
the band is checked admissible, and the oracle then continues from it."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

BAND = 1e-6


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_kv_realignment_amd as m
    return m


def _dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.view(dtype) if dtype is not None else t


def _bf16_bits(x32):
    """float32 -> bfloat16 bit patterns (round to nearest even), as uint16."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _admissible_draw(w, u, j):
    """Is id j an admissible inverse-CDF draw of weights w (fp64) for uniform u?"""
    c = np.cumsum(w)
    T = c[-1]
    t = float(u) * T
    lo = c[j - 1] if j > 0 else 0.0
    return w[j] > 0 and lo - BAND * T <= t < c[j] + BAND * T


def _admissible_cut(l, temperature, top_p, t):
    """Is t an admissible nucleus threshold of logits l: the mass at or above t
    reaches top_p and the mass strictly above it does not, within the band?"""
    e = oracle.softmax_row(l, temperature)
    lv = l.astype(np.float32) if l.dtype != np.uint16 else (l.astype(np.uint32) << 16).view(np.float32)
    if not np.isfinite(t) or not np.any(lv == t):
        return False
    at_or_above, above = e[lv >= t].sum(), e[lv > t].sum()
    return at_or_above >= top_p - BAND and above < top_p + BAND


def check_round(tl, dl, draft, u_acc, u_draw, temperature, acc, nxt, top_p=1.0, cut=None):
    """Every GPU decision against the oracle's arithmetic; returns the number of
    rows whose outcome differs from the oracle's (each one shown admissible).
    With top-p, `cut` holds the GPU's nucleus thresholds [B, 2D+1]: each one
    that differs from the oracle's must be admissible, and the oracle then
    decides with the GPU's thresholds."""
    B, D1, V = tl.shape
    D = D1 - 1
    if top_p < 1.0:
        _, _, _, ocut = oracle.verify_sample_logits(tl, dl, draft, u_acc, u_draw, temperature, top_p,
                                                    return_cut=True)
        for b, r in zip(*np.nonzero(cut != ocut)):
            row = tl[b, r] if r <= D else dl[b, r - D - 1]
            assert _admissible_cut(row, temperature, top_p, float(cut[b, r])), (b, r, cut[b, r], ocut[b, r])
    else:
        cut = np.full((B, 2 * D + 1), -np.inf, np.float32)
    oacc, onxt, _ = oracle.verify_sample_logits(tl, dl, draft, u_acc, u_draw, temperature, top_p, cut=cut)
    differ = 0
    for b in range(B):
        if acc[b] == oacc[b] and nxt[b] == onxt[b]:
            continue
        differ += 1
        a = int(acc[b])
        assert 0 <= a <= D
        def P(i):
            return oracle.softmax_row(tl[b, i], temperature, top_p, cut=cut[b, i])
        def Q(i):
            return oracle.softmax_row(dl[b, i], temperature, top_p, cut=cut[b, D + 1 + i])
        # acceptance decisions at positions 0..a (accept before a, reject at a < D)
        for i in range(min(a + 1, D)):
            x = int(draft[b, i])
            if not 0 <= x < V:
                assert i == a, "row %d: an out-of-range draft was accepted" % b
                continue
            p, q = P(i)[x], Q(i)[x]
            u = float(u_acc[b, i])
            ok = (u * q <= p) if q > 0 else (p > 0)
            if ok != (i < a):
                assert q > 0 and abs(u * q - p) <= BAND * p, "row %d: decision at %d outside the band" % (b, i)
        Pa = P(a)
        w = np.maximum(Pa - Q(a), 0.0) if a < D else Pa
        if not w.sum() > 0:
            w = Pa
        assert _admissible_draw(w, u_draw[b, a], int(nxt[b])), "row %d: draw outside the band" % b
    return differ


def _run(sd, tl, dl, draft, u_acc, u_draw, temperature, tdt=torch.float32, status=None, top_p=1.0,
         want_cut=False):
    if tdt == torch.bfloat16:
        t, d = _dev(_bf16_bits(tl), torch.bfloat16), _dev(_bf16_bits(dl), torch.bfloat16)
    else:
        np_dt = np.float16 if tdt == torch.float16 else np.float32
        t, d = _dev(tl.astype(np_dt)), _dev(dl.astype(np_dt))
    B, D1, _ = tl.shape
    cut = torch.full((B, 2 * D1 - 1), 7.0, dtype=torch.float32, device="cuda") if want_cut else None
    acc, nxt = sd.verify_sample_logits(t, d, _dev(draft), _dev(u_acc), _dev(u_draw), temperature, top_p=top_p,
                                       status=status, cutoff=cut)
    torch.cuda.synchronize()
    if want_cut:
        return acc.cpu().numpy(), nxt.cpu().numpy(), cut.cpu().numpy()
    return acc.cpu().numpy(), nxt.cpu().numpy()


def _host_logits(tl, tdt):
    """The logits exactly as the device reads them, in the form the oracle takes."""
    if tdt == torch.bfloat16:
        return _bf16_bits(tl)
    return tl.astype(np.float16 if tdt == torch.float16 else np.float32)


def test_stochastic_workload_from_logits(sd):
    """The stoch workload (B=32, D=8, V=32000, fp32 logits, temperature 0.8)."""
    cfg = synth.CONFIGS["stoch"]
    say("sample logits stoch")
    tl, dl, draft, u_acc, u_draw = synth.sampled_logits_round(cfg, 0)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt = _run(sd, tl, dl, draft, u_acc, u_draw, cfg.temperature, status=status)
    assert int(status.item()) == 0
    # each row that differs from the oracle has been shown admissible (within the band)
    assert check_round(tl, dl, draft, u_acc, u_draw, cfg.temperature, acc, nxt) <= 2
    assert acc.min() < cfg.D  # rejections and replacements happen


@pytest.mark.parametrize("seed", range(9))
def test_random_small(sd, seed):
    """Random shapes over several splits of 4096 logits and a ragged last split,
    D = 0, masked (-inf) logits, three temperatures and all three logit types."""
    rng = np.random.default_rng(700 + seed)
    tdt = [torch.float32, torch.float16, torch.bfloat16][seed % 3]
    B = int(rng.integers(1, 24))
    D = int(rng.integers(0, 7)) if seed % 4 else 0
    V = int([rng.integers(1, 50), rng.integers(1000, 5000), rng.integers(8000, 20000)][seed % 3])
    T = float([0.3, 1.0, 2.5][(seed // 3) % 3])
    say("sample logits random", seed, tdt, B, D, V, T)
    tl = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
    dl = (tl[:, :D] + rng.standard_normal((B, D, V)) * 0.5).astype(np.float32)
    if V > 3:
        tl[rng.random(tl.shape) < 0.05] = -np.inf
        dl[rng.random(dl.shape) < 0.05] = -np.inf
        tl[..., 0] = np.maximum(tl[..., 0], 0.0)  # every row keeps a finite logit
        dl[..., 0] = np.maximum(dl[..., 0], 0.0)
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    # half the drafts are the draft model's favourite, so acceptances happen
    fav = dl.argmax(-1) if D > 0 else np.zeros((B, 0), np.int64)
    pick = rng.random((B, D)) < 0.5
    draft[pick] = fav[pick]
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt = _run(sd, tl, dl, draft, u_acc, u_draw, T, tdt)
    h_t, h_d = _host_logits(tl, tdt), _host_logits(dl, tdt)
    check_round(h_t, h_d, draft, u_acc, u_draw, T, acc, nxt)


@pytest.mark.parametrize("shape", [(2, 255, 40), (600, 1, 300), (1, 255, 4100)])
def test_longest_draft_and_many_rows(sd, shape):
    """D = 255 (the longest draft; 511 rows of statistics per batch entry),
    many batch entries, and D = 255 with two splits of logits per row."""
    B, D, V = shape
    rng = np.random.default_rng(B + D + V)
    say("sample logits limits", shape)
    tl = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
    dl = (tl[:, :D] + rng.standard_normal((B, D, V)) * 0.3).astype(np.float32)
    draft = dl.argmax(-1).astype(np.int32)  # mostly accepted, so long prefixes are judged
    u_acc = (rng.random((B, D)) * 0.9).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt = _run(sd, tl, dl, draft, u_acc, u_draw, 1.0, torch.float32)
    check_round(tl, dl, draft, u_acc, u_draw, 1.0, acc, nxt)


def test_large_vocab_bf16(sd):
    """A 151936-entry bf16 vocabulary (38 splits)."""
    rng = np.random.default_rng(71)
    B, D, V, T = 4, 3, 151936, 0.9
    say("sample logits V=151936")
    tl = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
    dl = (tl[:, :D] + rng.standard_normal((B, D, V)) * 0.3).astype(np.float32)
    draft = dl.argmax(-1).astype(np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt = _run(sd, tl, dl, draft, u_acc, u_draw, T, torch.bfloat16)
    check_round(_bf16_bits(tl), _bf16_bits(dl), draft, u_acc, u_draw, T, acc, nxt)


def test_vanishing_temperature_is_greedy(sd):
    """At a temperature far below every logit gap the kernels make greedy
    verification's decisions (checked against the GPU greedy kernel)."""
    rng = np.random.default_rng(72)
    B, D, V = 24, 5, 5000
    say("sample logits T->0")
    tl = rng.permuted(np.tile(np.arange(V, dtype=np.float32), (B, D + 1, 1)), axis=2)
    dl = rng.permuted(np.tile(np.arange(V, dtype=np.float32), (B, D, 1)), axis=2)
    for b in range(B):
        for i in range(int(rng.integers(0, D + 1))):
            j, m = int(np.argmax(tl[b, i])), int(np.argmax(dl[b, i]))
            dl[b, i, [j, m]] = dl[b, i, [m, j]]
    draft = dl.argmax(-1).astype(np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt = _run(sd, tl, dl, draft, u_acc, u_draw, 1e-3)
    gacc, gnxt = sd.verify_greedy(_dev(tl), _dev(draft))
    assert np.array_equal(acc, gacc.cpu().numpy()) and np.array_equal(nxt, gnxt.cpu().numpy())
    assert acc.min() < D and acc.max() > 0


def test_worked_split_from_logits(sd):
    """The newsletter page's 40/60 example given as logits ln p, ln q."""
    say("sample logits worked split")
    tl = np.broadcast_to(np.log(np.array([0.4, 0.6])).astype(np.float32), (100, 2, 2)).copy()
    dl = np.broadcast_to(np.log(np.array([0.8, 0.2])).astype(np.float32), (100, 1, 2)).copy()
    drafts = np.array([0] * 80 + [1] * 20, np.int32)[:, None]
    u_acc = np.concatenate([(np.arange(80) + 0.5) / 80, (np.arange(20) + 0.5) / 20]).astype(np.float32)[:, None]
    u_draw = ((np.arange(200) + 0.5) / 200).astype(np.float32).reshape(100, 2)
    acc, nxt = _run(sd, tl, dl, drafts, u_acc, u_draw, 1.0)
    first = np.where(acc == 1, drafts[:, 0], nxt)
    assert int(np.sum(first == 0)) == 40 and int(np.sum(first == 1)) == 60


def test_out_of_range_draft_sets_status(sd):
    say("sample logits bad draft")
    rng = np.random.default_rng(73)
    B, D, V = 3, 4, 300
    tl = rng.standard_normal((B, D + 1, V)).astype(np.float32)
    dl = tl[:, :D].copy()  # q = p: every in-range draft is accepted
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    draft[1, 2] = V
    draft[2, 0] = -1
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt = _run(sd, tl, dl, draft, u_acc, u_draw, 1.0, status=status)
    assert int(status.item()) & sd.S_DRAFT_RANGE
    assert list(acc) == [D, 2, 0]
    check_round(tl, dl, draft, u_acc, u_draw, 1.0, acc, nxt)


def test_host_errors(sd):
    say("sample logits host errors")
    B, D, V = 2, 2, 64
    t = torch.zeros((B, D + 1, V), device="cuda")
    d = torch.zeros((B, D, V), device="cuda")
    dr = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    ua = torch.zeros((B, D), device="cuda")
    ud = torch.zeros((B, D + 1), device="cuda")
    for T, tp in ((0.0, 1.0), (-1.0, 1.0), (float("inf"), 1.0), (1.0, 0.0), (1.0, 1.5), (1.0, float("nan"))):
        with pytest.raises(sd.SpecDecError) as e:
            sd.verify_sample_logits(t, d, dr, ua, ud, T, top_p=tp)
        assert e.value.code == -1
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(sd.SpecDecError) as e:
        sd.verify_sample_logits(t, d, dr, ua, ud, 1.0, ws=small)
    assert e.value.code == -3
    with pytest.raises(ValueError):
        sd.verify_sample_logits(t, d.half(), dr, ua, ud, 1.0)
    # B = 0 is a no-op
    sd.verify_sample_logits(t[:0], d[:0], dr[:0], ua[:0], ud[:0], 1.0)
    torch.cuda.synchronize()


# ----------------------------------------------------------------------- top-p

@pytest.mark.parametrize("top_p", [0.9, 0.5])
def test_stochastic_workload_top_p(sd, top_p):
    """The stoch workload's logits with a nucleus on every row."""
    cfg = synth.CONFIGS["stoch"]
    say("sample logits stoch top_p", top_p)
    tl, dl, draft, u_acc, u_draw = synth.sampled_logits_round(cfg, 0)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt, cut = _run(sd, tl, dl, draft, u_acc, u_draw, cfg.temperature, status=status, top_p=top_p,
                         want_cut=True)
    assert int(status.item()) == 0
    *_, ocut = oracle.verify_sample_logits(tl, dl, draft, u_acc, u_draw, cfg.temperature, top_p, return_cut=True)
    assert np.mean(cut == ocut) > 0.98  # the thresholds agree outside the band
    assert check_round(tl, dl, draft, u_acc, u_draw, cfg.temperature, acc, nxt, top_p, cut) <= 1


@pytest.mark.parametrize("seed", range(9))
def test_top_p_random(sd, seed):
    """Random shapes, all three logit types, ties at every value (quantised
    logits), masked logits, D = 0 and top_p from 0.05 to 0.999."""
    rng = np.random.default_rng(900 + seed)
    tdt = [torch.float32, torch.float16, torch.bfloat16][seed % 3]
    B = int(rng.integers(1, 16))
    D = int(rng.integers(0, 6)) if seed % 4 else 0
    V = int([rng.integers(2, 60), rng.integers(1000, 5000), rng.integers(8000, 20000)][seed % 3])
    T = float([0.5, 1.0, 2.0][(seed // 3) % 3])
    top_p = float([0.05, 0.6, 0.9, 0.999][seed % 4])
    say("sample logits top_p random", seed, tdt, B, D, V, T, top_p)
    tl = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
    dl = (tl[:, :D] + rng.standard_normal((B, D, V)) * 0.5).astype(np.float32)
    if seed % 2 == 0:  # many ties
        tl, dl = np.round(tl * 2) / 2, np.round(dl * 2) / 2
    if V > 3:
        tl[rng.random(tl.shape) < 0.05] = -np.inf
        dl[rng.random(dl.shape) < 0.05] = -np.inf
        tl[..., 0] = np.maximum(tl[..., 0], 0.0)
        dl[..., 0] = np.maximum(dl[..., 0], 0.0)
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    fav = dl.argmax(-1) if D > 0 else np.zeros((B, 0), np.int64)
    pick = rng.random((B, D)) < 0.6
    draft[pick] = fav[pick]
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt, cut = _run(sd, tl, dl, draft, u_acc, u_draw, T, tdt, top_p=top_p, want_cut=True)
    h_t, h_d = _host_logits(tl, tdt), _host_logits(dl, tdt)
    check_round(h_t, h_d, draft, u_acc, u_draw, T, acc, nxt, top_p, cut)


@pytest.mark.parametrize("case", ["offset", "coarse_floats", "small_scale", "cold", "hot", "hot_bf16"])
def test_top_p_scales(sd, case):
    """Logit scales and temperatures at the edges of the selection's binning:
    logits near 3e4 and near 1e6 (float spacing as wide as, or wider than, a
    first-level bin, and many ties), logits of size 1e-3 at T = 1e-4, cold rows
    (T = 0.02: most masses round to 0) and hot rows (T = 50: hundreds of logits
    in the chosen first-level bin)."""
    rng = np.random.default_rng(97)
    B, D, V = 4, 3, 6007
    base = rng.standard_normal((B, D + 1, V))
    T, tdt = 1.0, torch.float32
    if case == "offset":
        tl = base * 2 + 3.0e4
    elif case == "coarse_floats":
        tl = base * 3 + 1.0e6
    elif case == "small_scale":
        tl, T = base * 1e-3, 1e-4
    elif case == "cold":
        tl, T = base * 2, 0.02
    else:
        tl, T = base * 2, 50.0
        tdt = torch.bfloat16 if case == "hot_bf16" else torch.float32
    tl = tl.astype(np.float32)
    dl = (tl[:, :D] + rng.standard_normal((B, D, V)) * (0.2 * float(tl.std()))).astype(np.float32)
    draft = dl.argmax(-1).astype(np.int32)
    draft[:, 1] = rng.integers(0, V, B)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    say("sample logits top_p scales", case)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt, cut = _run(sd, tl, dl, draft, u_acc, u_draw, T, tdt, status=status, top_p=0.9, want_cut=True)
    assert int(status.item()) == 0
    h_t, h_d = _host_logits(tl, tdt), _host_logits(dl, tdt)
    *_, ocut = oracle.verify_sample_logits(h_t, h_d, draft, u_acc, u_draw, T, 0.9, return_cut=True)
    assert np.mean(cut == ocut) > 0.9, case  # the thresholds agree outside the band
    check_round(h_t, h_d, draft, u_acc, u_draw, T, acc, nxt, 0.9, cut)


@pytest.mark.parametrize("case", ["random_f32", "flat_f32", "random_bf16"])
def test_max_vocab(sd, case):
    """The largest vocabulary the call takes, 2^22 ids: 1,024 statistics and
    mass splits per row, and with all target logits equal the nucleus's
    fixed-point total at its bound (2^22 masses of 2^41 units sum to 2^63);
    top_p 1 and 0.9."""
    rng = np.random.default_rng(99)
    B, D, V = 1, 2, 1 << 22
    tdt = torch.bfloat16 if case == "random_bf16" else torch.float32
    say("sample logits max vocab", case)
    if case == "flat_f32":
        tl = np.full((B, D + 1, V), 0.5, np.float32)
        dl = np.full((B, D, V), 0.5, np.float32)
        dl[..., : V // 2] = 0.25  # q below p on half the ids: a residual to draw from
    else:
        tl = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
        dl = (tl[:, :D] + rng.standard_normal((B, D, V)) * 0.5).astype(np.float32)
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    draft[0, 0] = int(np.argmax(dl[0, 0]))
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    h_t, h_d = _host_logits(tl, tdt), _host_logits(dl, tdt)
    for top_p in (1.0, 0.9):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        acc, nxt, cut = _run(sd, tl, dl, draft, u_acc, u_draw, 1.0, tdt, status=status, top_p=top_p, want_cut=True)
        assert int(status.item()) == 0, (case, top_p)
        if case == "flat_f32" and top_p < 1.0:  # every target id ties at the threshold
            assert np.all(cut[:, :D + 1] == 0.5)
        check_round(h_t, h_d, draft, u_acc, u_draw, 1.0, acc, nxt, top_p, cut if top_p < 1.0 else None)


def test_top_p_large_vocab_bf16(sd):
    """A 151936-entry bf16 vocabulary with top_p 0.9."""
    rng = np.random.default_rng(91)
    B, D, V, T = 4, 3, 151936, 0.9
    say("sample logits top_p V=151936")
    tl = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
    dl = (tl[:, :D] + rng.standard_normal((B, D, V)) * 0.3).astype(np.float32)
    draft = dl.argmax(-1).astype(np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt, cut = _run(sd, tl, dl, draft, u_acc, u_draw, T, torch.bfloat16, top_p=0.9, want_cut=True)
    check_round(_bf16_bits(tl), _bf16_bits(dl), draft, u_acc, u_draw, T, acc, nxt, 0.9, cut)


def test_vanishing_top_p_is_greedy(sd):
    """With a nucleus holding only each row's maximum (distinct logits), p and q
    are one-hot on the argmaxes, so sampled verification makes greedy
    verification's decisions (checked against the GPU greedy kernel)."""
    rng = np.random.default_rng(92)
    B, D, V = 24, 5, 3000
    say("sample logits top_p->0")
    tl = rng.permuted(np.tile(np.arange(V, dtype=np.float32) / 64, (B, D + 1, 1)), axis=2)
    dl = rng.permuted(np.tile(np.arange(V, dtype=np.float32) / 64, (B, D, 1)), axis=2)
    for b in range(B):
        for i in range(int(rng.integers(0, D + 1))):
            j, m = int(np.argmax(tl[b, i])), int(np.argmax(dl[b, i]))
            dl[b, i, [j, m]] = dl[b, i, [m, j]]
    draft = dl.argmax(-1).astype(np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt, cut = _run(sd, tl, dl, draft, u_acc, u_draw, 1.0, top_p=1e-6, want_cut=True)
    assert np.array_equal(cut[:, :D + 1], tl.max(-1)) and np.array_equal(cut[:, D + 1:], dl.max(-1))
    gacc, gnxt = sd.verify_greedy(_dev(tl), _dev(draft))
    assert np.array_equal(acc, gacc.cpu().numpy()) and np.array_equal(nxt, gnxt.cpu().numpy())
    assert acc.min() < D and acc.max() > 0


def test_no_nucleus_reports_minus_inf(sd):
    rng = np.random.default_rng(93)
    B, D, V = 3, 2, 500
    tl = rng.standard_normal((B, D + 1, V)).astype(np.float32)
    dl = rng.standard_normal((B, D, V)).astype(np.float32)
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    acc, nxt, cut = _run(sd, tl, dl, draft, rng.random((B, D)).astype(np.float32),
                         rng.random((B, D + 1)).astype(np.float32), 1.0, want_cut=True)
    assert np.all(cut == -np.inf)


@pytest.mark.parametrize("case", ["constant", "single_id", "two_values", "one_spike"])
def test_top_p_degenerate_rows(sd, case):
    """Rows the nucleus selection reaches in one step or at its edges: every
    logit equal (the nucleus is the whole row, ties at t all kept), a
    one-entry vocabulary, two values repeated over the row (t is the larger
    when its ids hold top_p), and one logit far above the rest (the nucleus
    is that id alone)."""
    rng = np.random.default_rng(95)
    B, D = 4, 3
    V = 1 if case == "single_id" else 3001
    say("sample logits top_p degenerate", case)
    if case == "constant":
        tl = np.full((B, D + 1, V), 1.25, np.float32)
    elif case == "single_id":
        tl = rng.standard_normal((B, D + 1, V)).astype(np.float32)
    elif case == "two_values":
        tl = np.where(rng.random((B, D + 1, V)) < 0.3, 2.0, -1.0).astype(np.float32)
    else:
        tl = rng.standard_normal((B, D + 1, V)).astype(np.float32)
        tl[..., 17] = 60.0
    dl = tl[:, :D].copy()
    dl[..., :V // 2] += 0.25 if V > 1 else 0.0
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    for top_p in (0.3, 0.999):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        acc, nxt, cut = _run(sd, tl, dl, draft, u_acc, u_draw, 1.0, status=status, top_p=top_p, want_cut=True)
        assert int(status.item()) == 0, (case, top_p)
        *_, ocut = oracle.verify_sample_logits(tl, dl, draft, u_acc, u_draw, 1.0, top_p, return_cut=True)
        assert np.array_equal(cut, ocut), (case, top_p)
        check_round(tl, dl, draft, u_acc, u_draw, 1.0, acc, nxt, top_p, cut)
        if case == "one_spike":  # the target rows' nucleus is the spike alone
            assert np.all(cut[:, :D + 1] == 60.0)
            assert np.all(nxt[acc == D] == 17)
