"""Pins of the oracle's pool lifecycle (finish at end-of-sequence or max length,
admit from a prompt queue): hand-worked cases, a per-sequence list model over
many random rounds of group / append / finish / admit, invariants of the slot
sets, and errors that change nothing."""
import numpy as np
import pytest

import oracle

EOS = 2


def _sets_ok(sched):
    act, fr = list(sched.active_list()), list(sched.free_list())
    assert sorted(act + fr) == list(range(sched.slots)) and len(set(act)) == len(act)
    assert fr == sorted(fr)


def test_finish_worked_example():
    """Slots 0..3; active [2, 0, 3], free [1].  After the append, slot 0 committed
    [7, EOS, 9] at positions 5..7 (finishes at length 7, dropping the 9); slot 3
    committed [4] at position 9 with max_len 10 (finishes at length 10); slot 2
    committed [5, 6] and goes on."""
    cap = 16
    tok = np.zeros((4, cap), np.int32)
    ln = np.array([8, 0, 4, 10], np.int32)
    tok[0, 5:8] = [7, EOS, 9]
    tok[2, 2:4] = [5, 6]
    tok[3, 9] = 4
    sched = oracle.Sched(4, active=[2, 0, 3])
    rows = np.array([0, 3, 2], np.int32)          # the round's batch order
    acc = np.array([2, 0, 1], np.int32)           # n = 3, 1, 2 committed
    retired = oracle.pool_finish(tok, ln, sched, rows, acc, D=4, eos_id=EOS, max_len=10)
    assert list(retired) == [0, 3]                # active-list order
    assert list(sched.active_list()) == [2]
    assert list(sched.free_list()) == [0, 1, 3]
    assert list(ln) == [7, 0, 4, 10]


def test_admit_worked_example():
    """Free slots [1, 3]; three queued prompts: prompts 0 and 1 go to slots 1 and
    3 (lowest first) and join the end of the active list; prompt 2 waits."""
    L, H, Dh, cap, pcap = 1, 2, 4, 12, 6
    rng = np.random.default_rng(0)
    kv = np.zeros((L, 2, 4, H, cap, Dh), np.float32)
    tok = np.zeros((4, cap), np.int32)
    ln = np.array([3, 0, 5, 0], np.int32)
    sched = oracle.Sched(4, active=[2, 0])
    pkv = rng.standard_normal((L, 2, 3, H, pcap, Dh)).astype(np.float32)
    ptok = rng.integers(10, 99, (3, pcap)).astype(np.int32)
    plen = np.array([4, 6, 2], np.int32)
    adm = oracle.pool_admit(kv, tok, ln, sched, pkv, ptok, plen)
    assert list(adm) == [1, 3]
    assert list(sched.active_list()) == [2, 0, 1, 3] and list(sched.free_list()) == [] and int(sched.q_head[0]) == 2
    assert list(ln) == [3, 4, 5, 6]
    assert np.array_equal(kv[:, :, 1, :, :4], pkv[:, :, 0, :, :4]) and np.all(kv[:, :, 1, :, 4:] == 0)
    assert np.array_equal(kv[:, :, 3, :, :6], pkv[:, :, 1])
    assert list(tok[1, :4]) == list(ptok[0, :4]) and list(tok[3, :6]) == list(ptok[1])
    # nothing left to fill: a second call admits nothing
    assert list(oracle.pool_admit(kv, tok, ln, sched, pkv, ptok, plen)) == []


def test_errors_change_nothing():
    cap = 8
    tok = np.zeros((3, cap), np.int32)
    ln = np.array([4, 4, 4], np.int32)
    sched = oracle.Sched(3, active=[0, 1])
    snap = (tok.copy(), ln.copy(), sched.copy())
    for rows, acc in (([0, 2], [0, 0]),           # slot 2 is not active
                      ([0, 0], [0, 0]),           # a slot twice
                      ([0, 1], [0, 5]),           # accepted length above D
                      ([0, 1], [0, 4])):          # more committed tokens than the length holds
        with pytest.raises(oracle.OracleError):
            oracle.pool_finish(tok, ln, sched, np.array(rows, np.int32), np.array(acc, np.int32), D=4, eos_id=EOS,
                               max_len=100)
        assert np.array_equal(tok, snap[0]) and np.array_equal(ln, snap[1])
        assert list(sched.active_list()) == [0, 1] and list(sched.free_list()) == [2]
    kv = np.zeros((1, 2, 3, 1, cap, 4), np.float32)
    with pytest.raises(oracle.OracleError) as e:  # a prompt longer than the pool's rows
        oracle.pool_admit(kv, tok, ln, sched, np.zeros((1, 2, 1, 1, 10, 4), np.float32), np.zeros((1, 10), np.int32),
                          np.array([9], np.int32))
    assert e.value.code == oracle.E_CAPACITY
    assert list(sched.free_list()) == [2] and int(sched.q_head[0]) == 0


class _Model:
    """Per-sequence list model of the pool: each slot a list of (token, kv
    position) pairs; the same policies written out with Python lists."""

    def __init__(self, slots):
        self.content = {s: [] for s in range(slots)}
        self.active, self.free, self.q_head = [], list(range(slots)), 0

    def admit(self, prompts):
        while self.free and self.q_head < len(prompts):
            s = min(self.free)
            self.free.remove(s)
            self.content[s] = list(prompts[self.q_head])
            self.active.append(s)
            self.q_head += 1

    def step(self, order, acc, draft, nxt, kvn, eos, max_len):
        """order: batch order (slots); kvn[j]: the entry's D+1 speculative KV rows."""
        gone = set()
        for j, s in enumerate(order):
            committed = list(draft[j, :acc[j]]) + [int(nxt[j])]
            c = len(self.content[s])
            self.content[s] += [(t, kvn[j][i]) for i, t in enumerate(committed)]
            for p in range(c, len(self.content[s])):
                if self.content[s][p][0] == eos or p + 1 >= max_len:
                    self.content[s] = self.content[s][:p + 1]
                    gone.add(s)
                    break
        retired = [s for s in self.active if s in gone]
        self.active = [s for s in self.active if s not in gone]
        self.free = sorted(self.free + retired)
        return retired


@pytest.mark.parametrize("seed", range(16))
def test_lifecycle_matches_list_model(seed):
    """Random pools run through rounds of group (over the active slots), append,
    finish and admit; every round the oracle's pool equals the list model."""
    rng = np.random.default_rng(500 + seed)
    slots = int(rng.integers(1, 12))
    G = int(rng.integers(1, 5))
    D = int(rng.integers(0, 4))
    L, H, Dh = 1, int(rng.integers(1, 3)), 4
    max_len = int(rng.integers(6, 30))
    cap = max_len + D + 1
    Q = int(rng.integers(0, 30))
    pcap = max_len
    plen = rng.integers(0, max_len, Q).astype(np.int32)
    pkv = rng.standard_normal((L, 2, Q, H, pcap, Dh)).astype(np.float32)
    ptok = rng.integers(3, 50, (Q, pcap)).astype(np.int32)
    prompts = [[(int(ptok[q, j]), pkv[:, :, q, :, j]) for j in range(plen[q])] for q in range(Q)]
    kv = np.zeros((L, 2, slots, H, cap, Dh), np.float32)
    tok = np.zeros((slots, cap), np.int32)
    ln = np.zeros(slots, np.int32)
    sched = oracle.Sched(slots, active=[])
    model = _Model(slots)
    oracle.pool_admit(kv, tok, ln, sched, pkv, ptok, plen)
    model.admit(prompts)
    for r in range(40):
        act = sched.active_list()
        assert list(act) == model.active
        _sets_ok(sched)
        if act.size == 0:
            break
        order, uni, wid, nu = oracle.group_by_len(ln[act], G)
        rows = act[order]
        B = rows.size
        acc = rng.integers(0, D + 1, B).astype(np.int32)
        draft = rng.integers(3, 50, (B, D)).astype(np.int32)
        nxt = rng.integers(3, 50, B).astype(np.int32)
        eos_at = rng.random((B, D)) < 0.1
        draft[eos_at] = EOS
        nxt[rng.random(B) < 0.1] = EOS
        kvn = rng.standard_normal((L, 2, B, H, D + 1, Dh)).astype(np.float32)
        oracle.append(kv, tok, ln, rows, kvn, draft, acc, nxt)
        retired = oracle.pool_finish(tok, ln, sched, rows, acc, D, EOS, max_len)
        want = model.step(list(rows), acc, draft, nxt, [[kvn[:, :, j, :, i] for i in range(D + 1)] for j in range(B)],
                          EOS, max_len)
        assert list(retired) == want
        oracle.pool_admit(kv, tok, ln, sched, pkv, ptok, plen)
        model.admit(prompts)
        for s in sched.active_list():
            content = model.content[int(s)]
            assert ln[s] == len(content)
            assert list(tok[s, :ln[s]]) == [t for t, _ in content]
            for j, (_, kvj) in enumerate(content):
                assert np.array_equal(kv[:, :, s, :, j], kvj)
