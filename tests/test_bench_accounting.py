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
