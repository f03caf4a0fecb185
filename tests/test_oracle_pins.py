"""Pins of the oracle against what the pages fix: their worked examples, closed
forms, special cases that reduce to library routines, and brute force."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _one_hot_logits(choices, V, base=0.0, peak=1.0):
    rows = np.full((len(choices), V), base, dtype=np.float32)
    for i, c in enumerate(choices):
        rows[i, c] = peak
    return rows


# ------------------------------------------------------------ worked examples

def test_greedy_commit_example():
    g = _load("greedy_commit.json")
    vocab = g["vocab"] + g["committed_text"]
    ids = {w: i for i, w in enumerate(vocab)}
    V = len(vocab)
    draft = np.array([ids[w] for w in g["draft"]], np.int32)
    D = len(draft)
    stated = {int(k): ids[v] for k, v in g["target_choice_stated"].items()}
    # position 4: the target agrees with the discarded draft 'gaming'; position 5: anything
    choices = [stated[0], stated[1], stated[2], ids["gaming"], ids["over"]]
    logits = _one_hot_logits(choices, V)[None]
    acc, nxt, tgt = oracle.verify_greedy(logits.reshape(D + 1, V), draft[None], 1, D, V)
    exp = g["expected"]
    assert acc[0] == exp["accepted_drafts"]
    assert vocab[nxt[0]] == exp["next_token"]
    a, committed = brute.greedy_one(logits[0], draft)
    assert a == exp["accepted_drafts"]
    assert [vocab[c] for c in committed] == exp["committed"]
    assert len(committed) == exp["committed_count"]

    # the same cycle through the EQSPEC realignment of a 1-row batch
    text = [ids[w] for w in g["committed_text"]]
    c0 = len(text)
    cap = 16
    tok = np.zeros((1, cap), np.int32)
    tok[0, :c0] = text
    mask = np.zeros((1, cap), np.int8)
    mask[0, :c0] = 1
    kv = np.zeros((1, 2, 1, 1, cap, 4), np.float32)
    kv_new = np.arange(1 * 2 * 1 * 1 * (D + 1) * 4, dtype=np.float32).reshape(1, 2, 1, 1, D + 1, 4)
    out = oracle.realign_eqspec(kv, kv_new, [c0], c0, tok, mask, acc, nxt, draft[None])
    assert out["width"] == len(exp["text_after"])
    assert [vocab[t] for t in out["tokens"][0, :out["width"]]] == exp["text_after"]


@pytest.mark.parametrize("case", _load("first_rejection.json")["cases"])
def test_first_rejection_cases(case):
    D = case["D"]
    V = 50
    rng = np.random.default_rng(7)
    choices = rng.integers(0, V, D + 1)
    draft = choices[:D].copy()
    r = case["first_rejected_position_1based"]
    if r is not None:
        k = r - 1
        draft[k] = (choices[k] + 1) % V  # the rejected draft; later drafts still agree with the target
    logits = _one_hot_logits(choices, V)
    acc, nxt, _ = oracle.verify_greedy(logits, draft[None], 1, D, V)
    a, committed = brute.greedy_one(logits, draft)
    exp = case["expected"]
    assert acc[0] == a == exp["accepted_drafts"]
    assert len(committed) == exp["committed_count"]
    assert 1 <= len(committed) <= D + 1
    assert nxt[0] == committed[-1] == choices[acc[0]]


def test_sampling_split_example():
    g = _load("sampling_split.json")
    p = np.array(g["p"], np.float32)
    q = np.array(g["q"], np.float32)
    nb, nl = g["draft_counts"]["battery"], g["draft_counts"]["life"]
    runs = g["runs"]
    assert nb + nl == runs
    # stratified acceptance uniforms: (k + 1/2)/n for each draft's n runs
    drafts = np.array([0] * nb + [1] * nl, np.int32)
    u_acc = np.concatenate([(np.arange(nb) + 0.5) / nb, (np.arange(nl) + 0.5) / nl]).astype(np.float32)
    u_draw = ((np.arange(runs * 2) + 0.5) / (runs * 2)).astype(np.float32).reshape(runs, 2)
    P = np.broadcast_to(p, (runs, 2, 2)).copy()
    Q = np.broadcast_to(q, (runs, 1, 2)).copy()
    acc, nxt, mass = oracle.verify_sample(P, Q, drafts[:, None], u_acc[:, None], u_draw)
    first = np.where(acc == 1, drafts, nxt)
    exp = g["expected"]
    assert int(np.sum(acc[:nb])) == exp["accepted_counts"]["battery"]
    assert int(np.sum(acc[nb:])) == exp["accepted_counts"]["life"]
    assert np.sum(acc[:nb]) / nb == exp["accept_fraction"]["battery"]
    assert np.sum(acc[nb:]) / nl == exp["accept_fraction"]["life"]
    # every rejected run is replaced by the residual's only token
    resid = np.maximum(p.astype(np.float64) - q, 0)
    assert np.allclose(resid / resid.sum(), exp["residual"])
    assert np.all(nxt[acc == 0] == 1)
    assert int(np.sum(first == 0)) == exp["final_counts"]["battery"]
    assert int(np.sum(first == 1)) == exp["final_counts"]["life"]
    for b in range(runs):
        a, committed = brute.sample_one(P[b], Q[b], drafts[b:b + 1], u_acc[b:b + 1], u_draw[b])
        assert (a, committed[-1]) == (acc[b], nxt[b])


# ------------------------------------------------------- sampled special cases

def _lib_inverse_cdf(w, u):
    c = np.cumsum(w.astype(np.float64))
    return int(np.searchsorted(c, float(u) * c[-1], side="right"))


def test_sample_p_equals_q_always_accepts():
    rng = np.random.default_rng(3)
    B, D, V = 64, 5, 40
    p = rng.random((B, D + 1, V)).astype(np.float32)
    p /= p.sum(-1, keepdims=True)
    q = p[:, :D].copy()
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt, _ = oracle.verify_sample(p, q, draft, u_acc, u_draw)
    assert np.all(acc == D)
    for b in range(B):
        assert nxt[b] == _lib_inverse_cdf(p[b, D], u_draw[b, D])


def test_sample_zero_target_mass_always_rejects_and_draws_from_p():
    rng = np.random.default_rng(4)
    B, D, V = 64, 3, 30
    p = rng.random((B, D + 1, V)).astype(np.float32)
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    for b in range(B):
        p[b, 0, draft[b, 0]] = 0.0
    q = np.zeros((B, D, V), np.float32)
    for b in range(B):
        for i in range(D):
            q[b, i, draft[b, i]] = 1.0
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt, mass = oracle.verify_sample(p, q, draft, u_acc, u_draw)
    assert np.all(acc == 0)
    for b in range(B):
        # residual max(0, p - onehot(x)) equals p because p(x) = 0
        assert nxt[b] == _lib_inverse_cdf(p[b, 0], u_draw[b, 0])
        assert mass[b] == pytest.approx(float(p[b, 0].astype(np.float64).sum()), rel=1e-12)


def test_sample_uniform_residual_is_floor_uV():
    B, V = 200, 64
    p = np.full((B, 1, V), 1.0 / V, np.float32)
    q = np.zeros((B, 0, V), np.float32)
    rng = np.random.default_rng(5)
    u = rng.random(B).astype(np.float32)
    keep = np.abs(u * V - np.round(u * V)) > 1e-3  # away from cell boundaries
    acc, nxt, _ = oracle.verify_sample(p, q, np.zeros((B, 0), np.int32), np.zeros((B, 0), np.float32), u[:, None])
    assert np.all(acc == 0)
    assert np.array_equal(nxt[keep], np.floor(u[keep].astype(np.float64) * V).astype(np.int32))


def test_sample_output_marginal_matches_target():
    """The first emitted token follows p and the acceptance rate is sum min(p, q)."""
    from scipy.stats import chisquare
    rng = np.random.default_rng(11)
    V, B = 6, 200_000
    p = rng.random(V) + 0.05
    p = (p / p.sum()).astype(np.float32)
    q = rng.random(V) + 0.05
    q = (q / q.sum()).astype(np.float32)
    P = np.broadcast_to(p, (B, 2, V)).copy()
    Q = np.broadcast_to(q, (B, 1, V)).copy()
    qq = q.astype(np.float64) / q.astype(np.float64).sum()
    draft = rng.choice(V, size=(B, 1), p=qq).astype(np.int32)
    u_acc = rng.random((B, 1)).astype(np.float32)
    u_draw = rng.random((B, 2)).astype(np.float32)
    acc, nxt, _ = oracle.verify_sample(P, Q, draft, u_acc, u_draw)
    first = np.where(acc == 1, draft[:, 0], nxt)
    counts = np.bincount(first, minlength=V)
    exp = p.astype(np.float64) / p.astype(np.float64).sum() * B
    assert chisquare(counts, exp).pvalue > 1e-3
    rate = float(np.minimum(p.astype(np.float64), qq).sum())
    sd = np.sqrt(rate * (1 - rate) / B)
    assert abs(acc.mean() - rate) < 5 * sd


# ---------------------------------------------------------- greedy tie rules

@pytest.mark.parametrize("enc", ["f32", "f16", "bf16"])
def test_greedy_ties_lowest_id_and_signed_zero(enc):
    V, D = 16, 2
    rows = np.full((D + 1, V), -3.0, np.float32)
    rows[0, [5, 2, 9]] = 1.5           # tie at the maximum: id 2 wins
    rows[1, :] = -1.0
    rows[1, 4] = -0.0                   # -0 and +0 compare equal: the lower id (4, holding -0) wins
    rows[1, 7] = 0.0
    rows[2, :] = -np.inf                # all -inf: id 0 wins
    if enc == "f32":
        enc_rows = rows
    elif enc == "f16":
        enc_rows = rows.astype(np.float16)
    else:
        enc_rows = (rows.view(np.uint32) >> 16).astype(np.uint16)
    draft = np.array([[2, 4]], np.int32)
    acc, nxt, tgt = oracle.verify_greedy(enc_rows, draft, 1, D, V)
    assert list(tgt[0]) == [2, 4, 0]
    assert acc[0] == 2 and nxt[0] == 0


def test_greedy_matches_brute_on_discrete_logits():
    rng = np.random.default_rng(21)
    for trial in range(200):
        B = int(rng.integers(1, 6))
        D = int(rng.integers(0, 6))
        V = int(rng.integers(1, 12))
        vals = np.array([-2.0, -0.0, 0.0, 1.0, 1.0, 3.0], np.float32)
        logits = vals[rng.integers(0, len(vals), (B * (D + 1), V))]
        tgt_first = np.argmax(logits.reshape(B, D + 1, V), axis=-1)
        draft = np.where(rng.random((B, D)) < 0.7, tgt_first[:, :D], rng.integers(0, V, (B, D))).astype(np.int32)
        acc, nxt, _ = oracle.verify_greedy(logits, draft, B, D, V)
        for b in range(B):
            a, committed = brute.greedy_one(logits[b * (D + 1):(b + 1) * (D + 1)], draft[b])
            assert (a, committed[-1]) == (acc[b], nxt[b])


def test_sample_matches_brute_random():
    rng = np.random.default_rng(22)
    for trial in range(60):
        B = int(rng.integers(1, 5))
        D = int(rng.integers(0, 5))
        V = int(rng.integers(1, 9))
        p = rng.random((B, D + 1, V)).astype(np.float32)
        p[rng.random(p.shape) < 0.2] = 0.0
        p[..., 0] += 0.01
        p /= p.sum(-1, keepdims=True)
        q = rng.random((B, D, V)).astype(np.float32)
        q[rng.random(q.shape) < 0.2] = 0.0
        q[..., -1] += 0.01
        q /= q.sum(-1, keepdims=True)
        draft = rng.integers(0, V, (B, D)).astype(np.int32)
        u_acc = rng.random((B, D)).astype(np.float32)
        u_draw = rng.random((B, D + 1)).astype(np.float32)
        acc, nxt, _ = oracle.verify_sample(p, q, draft, u_acc, u_draw)
        for b in range(B):
            a, committed = brute.sample_one(p[b], q[b], draft[b], u_acc[b], u_draw[b])
            assert (a, committed[-1]) == (acc[b], nxt[b]), (trial, b)
