"""Pins of the oracle's sampled verification from logits (temperature and
top-p), against what the pages and the mathematics fix: the pages' 40/60
worked example rebuilt from logits, the limit of a vanishing temperature
(which is greedy verification, pinned on its own), uniform and two-token
closed forms, invariances of the softmax, nucleus examples worked by hand
(ties included), and the output distribution of speculative sampling."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32(x):
    return np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------- softmax rows

def test_softmax_uniform_logits():
    for V in (1, 7, 1000):
        p = oracle.softmax_row(np.full(V, 3.25, np.float32), 0.8)
        assert np.all(p == 1.0 / V)


def test_softmax_two_tokens_closed_form():
    # logits 0 and T*ln(3): probabilities 1/4 and 3/4
    T = 0.5
    p = oracle.softmax_row(_f32([0.0, T * np.log(3.0)]), T)
    lg = float(np.float32(T * np.log(3.0)))
    want1 = 1.0 / (1.0 + np.exp(-lg / T))
    assert p[1] == pytest.approx(0.75, rel=1e-7)
    assert p[1] == pytest.approx(want1, rel=1e-14)
    assert p.sum() == pytest.approx(1.0, rel=1e-15)


def test_softmax_shift_and_temperature_scaling():
    rng = np.random.default_rng(1)
    l = rng.integers(-40, 40, 500).astype(np.float32)  # integer logits: shifts and doubling are exact
    base = oracle.softmax_row(l, 0.8)
    assert np.array_equal(oracle.softmax_row(l + np.float32(1024.0), 0.8), base)
    assert np.array_equal(oracle.softmax_row(l * np.float32(2.0), 1.6), base)
    # a larger temperature flattens: the top probability falls, the lowest rises
    hot = oracle.softmax_row(l, 8.0)
    assert hot.max() < base.max() and hot.min() > base.min()


@pytest.mark.parametrize("enc", ["f16", "bf16"])
def test_softmax_half_precision_logits_widen_exactly(enc):
    rng = np.random.default_rng(2)
    l32 = (rng.standard_normal(300) * 2).astype(np.float32)
    if enc == "f16":
        half = l32.astype(np.float16)
        wide = half.astype(np.float32)
    else:
        bits = (l32.view(np.uint32) >> 16).astype(np.uint16)  # truncation gives a valid bf16 value
        half = bits
        wide = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(oracle.softmax_row(half, 0.7), oracle.softmax_row(wide, 0.7))


# ----------------------------------------------------------------------- top-p

def test_top_p_worked_nucleus():
    probs = np.array([0.05, 0.5, 0.15, 0.3])
    l = np.log(probs).astype(np.float32)
    # sorted masses 0.5, 0.3, 0.15, 0.05: cumulative 0.5, 0.8, 0.95, 1.0
    p = oracle.softmax_row(l, 1.0, top_p=0.7)
    assert np.allclose(p, [0.0, 0.5 / 0.8, 0.0, 0.3 / 0.8], rtol=1e-6, atol=0)
    p = oracle.softmax_row(l, 1.0, top_p=0.9)
    assert np.allclose(p, [0.0, 0.5 / 0.95, 0.15 / 0.95, 0.3 / 0.95], rtol=1e-6, atol=0)
    p = oracle.softmax_row(l, 1.0, top_p=0.4)
    assert np.array_equal(p, [0.0, 1.0, 0.0, 0.0])
    assert np.array_equal(oracle.softmax_row(l, 1.0, top_p=1.0), oracle.softmax_row(l, 1.0))


def test_top_p_keeps_every_tie_at_the_cutoff():
    l = np.log(np.array([0.3, 0.4, 0.3])).astype(np.float32)
    assert l[0] == l[2]
    # 0.4 alone is short of 0.5; the next value (0.3) is held by ids 0 and 2, both kept
    p = oracle.softmax_row(l, 1.0, top_p=0.5)
    assert np.all(p > 0) and p.sum() == pytest.approx(1.0, rel=1e-15)
    assert np.array_equal(p, oracle.softmax_row(l, 1.0))


def test_top_p_reported_and_forced_cutoff():
    """The threshold the oracle applies is the hand-worked one (the 0.3 logit at
    top_p 0.7, the 0.15 logit at 0.9, -inf when every id is kept), and forcing
    a threshold forms exactly that nucleus."""
    probs = np.array([0.05, 0.5, 0.15, 0.3])
    l = np.log(probs).astype(np.float32)
    TL = np.broadcast_to(l, (4, 1, 4)).copy()
    DL = np.zeros((4, 0, 4), np.float32)
    draft = np.zeros((4, 0), np.int32)
    ua = np.zeros((4, 0), np.float32)
    ud = np.full((4, 1), 0.5, np.float32)
    for tp, want in ((0.7, l[3]), (0.9, l[2]), (0.4, l[1]), (1.0, -np.inf)):
        *_, used = oracle.verify_sample_logits(TL, DL, draft, ua, ud, 1.0, top_p=tp, return_cut=True)
        assert np.all(used == want), (tp, used)
    # a forced threshold overrides top_p: the 0.15 logit keeps three ids
    assert np.array_equal(oracle.softmax_row(l, 1.0, top_p=0.7, cut=l[2]), oracle.softmax_row(l, 1.0, top_p=0.9))
    assert np.array_equal(oracle.softmax_row(l, 1.0, top_p=0.5, cut=-np.inf), oracle.softmax_row(l, 1.0))
    # verification with the thresholds it computed itself is unchanged
    rng = np.random.default_rng(17)
    B, D, V = 6, 3, 400
    tl = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
    dl = (tl[:, :D] + rng.standard_normal((B, D, V)) * 0.5).astype(np.float32)
    dr = dl.argmax(-1).astype(np.int32)
    u1 = rng.random((B, D)).astype(np.float32)
    u2 = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt, mass, used = oracle.verify_sample_logits(tl, dl, dr, u1, u2, 0.8, top_p=0.85, return_cut=True)
    assert np.all(np.isfinite(used))
    acc2, nxt2, mass2 = oracle.verify_sample_logits(tl, dl, dr, u1, u2, 0.8, top_p=0.3, cut=used)
    assert np.array_equal(acc, acc2) and np.array_equal(nxt, nxt2) and np.array_equal(mass, mass2)


def test_top_p_invalid_settings_rejected():
    for T, tp in ((0.0, 1.0), (-1.0, 1.0), (np.inf, 1.0), (1.0, 0.0), (1.0, 1.5)):
        with pytest.raises(oracle.OracleError):
            oracle.softmax_row(_f32([0.0, 1.0]), T, top_p=tp)


# ---------------------------------------------------------- sampled verification

def test_pages_split_example_from_logits():
    """The 40/60 example with p and q given by logits ln p, ln q at temperature 1."""
    g = json.load(open(os.path.join(GOLD, "sampling_split.json")))
    p, q = np.array(g["p"]), np.array(g["q"])
    nb, nl = g["draft_counts"]["battery"], g["draft_counts"]["life"]
    runs = nb + nl
    drafts = np.array([0] * nb + [1] * nl, np.int32)
    u_acc = np.concatenate([(np.arange(nb) + 0.5) / nb, (np.arange(nl) + 0.5) / nl]).astype(np.float32)
    u_draw = ((np.arange(runs * 2) + 0.5) / (runs * 2)).astype(np.float32).reshape(runs, 2)
    tl = np.broadcast_to(np.log(p).astype(np.float32), (runs, 2, 2)).copy()
    dl = np.broadcast_to(np.log(q).astype(np.float32), (runs, 1, 2)).copy()
    acc, nxt, _ = oracle.verify_sample_logits(tl, dl, drafts[:, None], u_acc[:, None], u_draw, 1.0)
    exp = g["expected"]
    assert int(acc[:nb].sum()) == exp["accepted_counts"]["battery"]
    assert int(acc[nb:].sum()) == exp["accepted_counts"]["life"]
    assert np.all(nxt[acc == 0] == 1)
    first = np.where(acc == 1, drafts, nxt)
    assert int((first == 0).sum()) == exp["final_counts"]["battery"]
    assert int((first == 1).sum()) == exp["final_counts"]["life"]


@pytest.mark.parametrize("top_p", [1.0, 0.9])
def test_vanishing_temperature_is_greedy(top_p):
    """At a temperature far below every logit gap p and q are one-hot at the
    argmax, so sampled verification makes greedy verification's decisions for
    any uniforms."""
    rng = np.random.default_rng(7)
    B, D, V = 40, 5, 300
    tl = rng.permuted(np.tile(np.arange(V, dtype=np.float32), (B, D + 1, 1)), axis=2)  # distinct integer logits
    dl = rng.permuted(np.tile(np.arange(V, dtype=np.float32), (B, D, 1)), axis=2)
    # plant: the draft's argmax equals the target's at a random prefix of positions
    for b in range(B):
        k = rng.integers(0, D + 1)
        for i in range(k):
            j = int(np.argmax(tl[b, i]))
            m = int(np.argmax(dl[b, i]))
            dl[b, i, [j, m]] = dl[b, i, [m, j]]
    draft = dl.argmax(axis=2).astype(np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt, _ = oracle.verify_sample_logits(tl, dl, draft, u_acc, u_draw, 1e-3, top_p=top_p)
    gacc, gnxt, _ = oracle.verify_greedy(tl.reshape(B * (D + 1), V), draft, B, D, V)
    assert np.array_equal(acc, gacc) and np.array_equal(nxt, gnxt)
    assert acc.min() < D < acc.max() + 1  # both outcomes occur


def test_matches_probability_oracle_away_from_boundaries():
    """Feeding the fp32-rounded softmax to the probability oracle gives the same
    decisions wherever no decision lies within 1e-4 of its threshold."""
    rng = np.random.default_rng(9)
    B, D, V, T = 200, 4, 64, 0.8
    tl = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
    dl = (tl[:, :D] + rng.standard_normal((B, D, V)) * 0.5).astype(np.float32)
    P = np.stack([[oracle.softmax_row(tl[b, i], T) for i in range(D + 1)] for b in range(B)])
    Q = np.stack([[oracle.softmax_row(dl[b, i], T) for i in range(D)] for b in range(B)])
    draft = np.array([[rng.choice(V, p=Q[b, i]) for i in range(D)] for b in range(B)], np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt, _ = oracle.verify_sample_logits(tl, dl, draft, u_acc, u_draw, T)
    pacc, pnxt, _ = oracle.verify_sample(P.astype(np.float32), Q.astype(np.float32), draft, u_acc, u_draw)
    compared = 0
    for b in range(B):
        ratios = [P[b, i, draft[b, i]] / Q[b, i, draft[b, i]] for i in range(D)]
        if any(abs(u_acc[b, i] - r) < 1e-4 * max(r, 1e-30) for i, r in enumerate(ratios)):
            continue
        a = acc[b]
        w = np.maximum(P[b, a] - Q[b, a], 0) if a < D else P[b, D]
        c = np.cumsum(w)
        if np.min(np.abs(c - u_draw[b, a] * c[-1])) < 1e-4 * c[-1]:
            continue
        assert (acc[b], nxt[b]) == (pacc[b], pnxt[b]), b
        compared += 1
    assert compared > 0.9 * B


@pytest.mark.parametrize("top_p", [1.0, 0.8])
def test_output_marginal_matches_target(top_p):
    """The first emitted token follows p (after temperature and top-p) and the
    acceptance rate is sum(min(p, q))."""
    from scipy.stats import chisquare
    rng = np.random.default_rng(13)
    V, B, T = 6, 200_000, 0.7
    tl = (rng.standard_normal(V)).astype(np.float32)
    dl = (tl + rng.standard_normal(V) * 0.8).astype(np.float32)
    p = oracle.softmax_row(tl, T, top_p)
    q = oracle.softmax_row(dl, T, top_p)
    draft = rng.choice(V, size=(B, 1), p=q).astype(np.int32)
    u_acc = rng.random((B, 1)).astype(np.float32)
    u_draw = rng.random((B, 2)).astype(np.float32)
    TL = np.broadcast_to(tl, (B, 2, V)).copy()
    DL = np.broadcast_to(dl, (B, 1, V)).copy()
    acc, nxt, _ = oracle.verify_sample_logits(TL, DL, draft, u_acc, u_draw, T, top_p=top_p)
    first = np.where(acc == 1, draft[:, 0], nxt)
    counts = np.bincount(first, minlength=V)
    keep = p > 0
    assert np.all(counts[~keep] == 0)
    assert chisquare(counts[keep], p[keep] / p[keep].sum() * B).pvalue > 1e-3
    rate = float(np.minimum(p, q).sum())
    assert abs(acc.mean() - rate) < 5 * np.sqrt(rate * (1 - rate) / B)
