"""Per-sequence brute force, the second reference (TEST INFRASTRUCTURE ONLY).

One sequence at a time, no batch, no padding: the plain statement of what a
verification cycle commits and what the sequence's state becomes.  Written
independently of oracle.c (numpy routines, exact rational comparisons) so the
two can pin each other on small inputs.

Passages: "Inference Engineering Part 5/8: When Speculative Decoding Backfires",
sections "Draft Possible Tokens, Then Verify Them Together" and "Exactness Means
Different Things For Greedy And Sampled Output" (the acceptance rules and the
1..D+1 committed tokens), section "Acceptance changes across the workload"
(committed KV kept, speculative KV committed or discarded); "Batch Speculative
Decoding Done Right" section 1 (batched output must equal unbatched output).
"""
from fractions import Fraction

import numpy as np


def greedy_one(logit_rows, draft):
    """logit_rows [D+1, V] (any real dtype), draft [D] -> (accepted, committed ids).

    numpy.argmax returns the first occurrence of the maximum (lowest id on ties).
    """
    rows = np.asarray(logit_rows, dtype=np.float64)
    D = len(draft)
    choice = [int(np.argmax(rows[i])) for i in range(D + 1)]
    a = 0
    for i in range(D):
        if int(draft[i]) != choice[i]:
            break
        a += 1
    return a, [int(x) for x in draft[:a]] + [choice[a]]


def sample_one(p, q, draft, u_accept, u_draw):
    """p [D+1,V], q [D,V] float32 -> (accepted, committed ids).

    Acceptance u <= p/q is decided with exact rationals; the replacement (or the
    bonus) is the inverse CDF of normalize(max(0, p - q)) (or of p at position D)
    via numpy cumsum + searchsorted: the first id whose cumulative mass exceeds u
    times the total.
    """
    D = len(draft)
    V = p.shape[1]
    a = D
    for i in range(D):
        x = int(draft[i])
        px, qx = Fraction(float(p[i, x])), Fraction(float(q[i, x]))
        u = Fraction(float(u_accept[i]))
        ok = (u * qx <= px) if qx > 0 else (px > 0)
        if not ok:
            a = i
            break
    if a < D:
        w = np.maximum(p[a].astype(np.float64) - q[a].astype(np.float64), 0.0)
    else:
        w = p[D].astype(np.float64)
    if not w.sum() > 0:
        w = np.maximum(p[a].astype(np.float64), 0.0)
    c = np.cumsum(w)
    j = int(np.searchsorted(c, float(u_draw[a]) * c[-1], side="right"))
    if j >= V:
        j = int(np.nonzero(w > 0)[0][-1])
    return a, [int(x) for x in draft[:a]] + [j]


def advance(tokens, kv, committed, kv_new):
    """State of one sequence after a cycle: tokens ++ committed, and the KV of
    its content ++ the first len(committed) speculative entries.

    tokens: list of ids; kv [L,2,H,c,Dh]; kv_new [L,2,H,D+1,Dh]."""
    n = len(committed)
    return list(tokens) + list(committed), np.concatenate([kv, kv_new[:, :, :, :n, :]], axis=3)


def chain_final(kv0, lens0, width0, kv_new_rounds, acc_rounds, left_pad=True):
    """KV of a batch after a chain of rounds, one sequence at a time: each row's
    content is its initial content followed by the first a+1 speculative entries
    of every round, in round order (advance() applied round after round, written
    as one concatenation per row).  The rows are then laid out as the batch
    stores them: left-padded to the longest (a rectangle) or left-aligned (a
    pool), zero elsewhere.

    kv0 [L,2,B,H,cap,Dh] holds row b's content at [width0 - lens0[b], width0)
    (left_pad) or [0, lens0[b]) (a pool); kv_new_rounds[r] [L,2,B,H,D+1,Dh];
    acc_rounds[r] [B].  Returns (kv [L,2,B,H,W,Dh], lens [B], W) with W the
    longest final length."""
    L, _, B, H, _, Dh = kv0.shape
    seqs = []
    for b in range(B):
        c = int(lens0[b])
        lo = width0 - c if left_pad else 0
        parts = [kv0[:, :, b, :, lo:lo + c]]
        for kvn, acc in zip(kv_new_rounds, acc_rounds):
            parts.append(kvn[:, :, b, :, :int(acc[b]) + 1])
        seqs.append(np.concatenate(parts, axis=3))
    lens = np.array([s.shape[3] for s in seqs], dtype=np.int32)
    W = int(lens.max()) if B else 0
    out = np.zeros((L, 2, B, H, W, Dh), dtype=kv0.dtype)
    for b, s in enumerate(seqs):
        if left_pad:
            out[:, :, b, :, W - s.shape[3]:] = s
        else:
            out[:, :, b, :, :s.shape[3]] = s
    return out, lens, W
