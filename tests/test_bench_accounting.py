"""bench.py's algorithmic-byte model agrees with what the oracle actually moves:
the lengths and widths it replays from the accepted-length history are the
oracle's, and its KV byte count equals old content + committed entries read and
the full new rectangle written."""
import numpy as np

import bench
import oracle
import synth


def test_round_bytes_match_oracle_rounds():
    cfg = synth.CONFIGS["8b-gqa"]
    lens = synth.lengths(cfg)
    S = int(lens.max())
    tok, pos, mask = synth.tokens_host(cfg, lens, S, True)
    kv = synth.kv_host(cfg, lens, S, True, layer0=0, nlayers=1)
    accs, expect = [], []
    lens0 = lens.copy()
    for r in range(3):
        plant, _, draft = synth.plan_greedy(cfg, r)
        acc, nxt, _ = oracle.verify_greedy(synth.logits_host(cfg, r, plant), draft, cfg.B, cfg.D, cfg.V)
        out = oracle.realign_eqspec(kv, synth.kvnew_host(cfg, r, 0, 1), lens, S, tok, mask, acc, nxt, draft)
        W = out["width"]
        # positions read (old content + committed entries) and written (the new rectangle), per layer slab
        read_pos = int(lens.sum()) + int((acc + 1).sum())
        expect.append(cfg.kv_pos_bytes * (read_pos + cfg.B * W))
        accs.append(acc)
        kv, lens, S, tok, mask = out["kv"], out["len"], W, out["tokens"], out["mask"]
    vb, rb = bench.round_bytes(cfg, lens0, int(lens0.max()), np.array(accs))
    meta = rb - np.array(expect, dtype=np.float64)
    assert np.all(meta > 0) and np.all(meta < 1e6)  # token/position/mask bytes only
    assert np.all(vb == cfg.B * cfg.D1 * cfg.V * 2 + cfg.B * cfg.D * 4 + 8 * cfg.B)


def test_round_bytes_inplace_position_count():
    """In-place byte model against a per-position walk of the oracle's rounds:
    a position of [0, S') is written when its new content is not already there
    (moved content, committed entries, pad where content or unused capacity
    was), and read when it is moved content or a committed entry."""
    cfg = synth.CONFIGS["8b-gqa"]
    lens = synth.lengths(cfg)
    S = int(lens.max())
    tok, pos, mask = synth.tokens_host(cfg, lens, S, True)
    kv = synth.kv_host(cfg, lens, S, True, layer0=0, nlayers=1)
    accs, expect = [], []
    lens0 = lens.copy()
    for r in range(3):
        plant, _, draft = synth.plan_greedy(cfg, r)
        acc, nxt, _ = oracle.verify_greedy(synth.logits_host(cfg, r, plant), draft, cfg.B, cfg.D, cfg.V)
        out = oracle.realign_eqspec(kv, synth.kvnew_host(cfg, r, 0, 1), lens, S, tok, mask, acc, nxt, draft)
        W = out["width"]
        moved_bytes = 0
        for b in range(cfg.B):
            c, n = int(lens[b]), int(acc[b]) + 1
            old_start, new_start = S - c, W - c - n
            reads = writes = 0
            for j in range(W):
                k = j - new_start  # index into the row's new content, < 0 on pad
                if k < 0:
                    writes += j >= old_start  # pad where old content (or unused capacity) was
                elif k < c:
                    if new_start != old_start:
                        reads += 1
                        writes += 1
                else:
                    reads += 1
                    writes += 1
            moved_bytes += cfg.kv_pos_bytes * (reads + writes)
        expect.append(moved_bytes)
        accs.append(acc)
        kv, lens, S, tok, mask = out["kv"], out["len"], W, out["tokens"], out["mask"]
    rb = bench.round_bytes_inplace(cfg, lens0, int(lens0.max()), np.array(accs))
    meta = rb - np.array(expect, dtype=np.float64)
    assert np.all(meta > 0) and np.all(meta < 1e6)  # token/position/mask bytes only
    _, full = bench.round_bytes(cfg, lens0, int(lens0.max()), np.array(accs))
    assert np.all(rb < full)


def test_round_bytes_paged_counts_written_slots():
    """Paged byte model: the KV part is the committed entries read once and
    written once; the slots the oracle's paged append changes are exactly
    those entries, and the rest of the model is metadata."""
    cfg = synth.CONFIGS["8b-gqa"]
    page = bench.PAGE
    lens = synth.lengths(cfg)
    S = int(lens.max())
    tok, _, _ = synth.tokens_host(cfg, lens, S, True)
    kv = synth.kv_host(cfg, lens, S, True, layer0=0, nlayers=1)
    mb = -(-cfg.cap // page)
    st = oracle.PagedState(1, cfg.H, cfg.Dh, cfg.B * mb, page, mb, cfg.B, kv.dtype)
    cap = max(cfg.cap, S)
    kvc = np.zeros(kv.shape[:4] + (cap, cfg.Dh), kv.dtype)
    kvc[..., :kv.shape[4], :] = kv
    tokc = np.zeros((cfg.B, cap), np.int32)
    tokc[:, :tok.shape[1]] = tok
    oracle.paged_admit(st, kvc, tokc, lens, S)
    accs, written = [], []
    for r in range(3):
        plant, _, draft = synth.plan_greedy(cfg, r)
        acc, nxt, _ = oracle.verify_greedy(synth.logits_host(cfg, r, plant), draft, cfg.B, cfg.D, cfg.V)
        before = st.pages.copy()
        oracle.paged_append(st, synth.kvnew_host(cfg, r, 0, 1), draft, acc, nxt)
        slots = np.any(before.view(np.uint16) != st.pages.view(np.uint16), axis=(0, 1, 3, 5))
        written.append(int(slots.sum()))
        accs.append(acc)
        assert written[-1] == int((acc + 1).sum())
    pb = bench.round_bytes_paged(cfg, lens, np.array(accs), page)
    kv_part = 2 * cfg.kv_pos_bytes * np.array(written, dtype=np.float64)
    meta = pb - kv_part
    assert np.all(meta > 0) and np.all(meta < 1e6)


def test_cpu_baseline_reports_both_oracle_builds():
    """The benchmark's CPU leg on the tiny workload: the single-threaded
    oracle's rate as the value (one core), the OpenMP build's beside it, and
    the threaded build switched off again afterwards."""
    cfg = synth.CONFIGS["tiny"]
    lens = synth.lengths(cfg)
    S = int(lens.max())
    tok, pos, mask = synth.tokens_host(cfg, lens, S, True)
    plans = [synth.plan_greedy(cfg, r) for r in range(3)]
    cpu = bench.cpu_baseline(cfg, plans, lens, S, tok, mask, 3, cfg.L)
    assert cpu["value"] > 0 and cpu["cores"] == 1 and cpu["kind"] == "oracle" and cpu["unit"] == "rounds/s"
    assert cpu["all_cores"]["value"] > 0 and cpu["all_cores"]["cores"] >= 1
    assert oracle.threads() == 1


def test_cycle_stats_histogram_and_rates():
    import numpy as np
    import bench
    acc = np.array([[0, 5, 2], [5, 5, 1]])  # 2 rounds x 3 rows, D = 5
    c = bench.cycle_stats(acc, 5, rounds_per_s=10.0)
    assert c["accept_len_histogram"] == [1, 1, 1, 0, 0, 3]
    assert c["first_rejection_position_histogram"] == [1, 1, 1, 0, 0] and c["no_rejection_rows"] == 3
    assert c["accepted_drafts_per_round"] == 9.0                 # (0+5+2 + 5+5+1) / 2
    assert c["committed_tokens_per_round"] == 12.0               # (1+6+3 + 6+6+2) / 2
    assert c["committed_tokens_per_round_min_max"] == [10, 14]
    assert c["committed_tokens_per_s"] == 120.0


def test_host_info_reports_cpus_and_ram():
    import bench
    h = bench.host_info()
    assert h["cpu_count"] >= 1 and h["ram_bytes"] > 0
