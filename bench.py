#!/usr/bin/env python3
"""Benchmark of the verify-and-resynchronize step on one MI355X.

A step is one round of batch speculative decoding's hot path on the 8B-GQA
shaped workload: greedy verification of B=16 rows x D=5 drafts against bf16
logits [16, 6, 151936], then the EQSPEC unpad-append-repad of a bf16 KV cache
of 36 layers x 8 KV heads x 128 (lengths uniform in [256, 2048], left-padded)
with fresh seeded KV entries for the committed tokens.  Rounds are chained:
each realigns the previous round's output.  All inputs are synthetic and
already resident in HBM when timing starts; every round has its own logits
buffer, so nothing is re-read from cache across rounds.

Prints one JSON line: rounds/s over the timed rounds, the realign kernel's
achieved HBM bandwidth against the 8 TB/s peak (per-launch HIP events on the
launch stream), and the CPU oracle timed on a bounded sample of the same
workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify+realign rounds/sec and realign HBM GB/s (% of peak) at B=16"
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "realign_eqspec_8b_gqa_traffic.txt")
REALIGN_SRC = os.path.join(ROOT, "ragged_kv_realignment_amd", "csrc", "realign.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed chained rounds")
    ap.add_argument("--warmup", type=int, default=8, help="untimed rounds before the timed chain")
    ap.add_argument("--config", default="8b-gqa")
    ap.add_argument("--cpu-rounds", type=int, default=64, help="oracle sample: rounds")
    ap.add_argument("--cpu-layers", type=int, default=36, help="oracle sample: KV layers realigned (scaled to all)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--copy-calib-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration for profiling)")
    return ap.parse_args()


def realign_kernel_sha():
    with open(REALIGN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_per_launch():
    """HBM bytes per realign launch from the committed counter summary, or None
    when it is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m_sha = re.search(r"^kernel_source_sha256_16:\s*(\w+)", txt, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not m_sha or not m_b or m_sha.group(1) != realign_kernel_sha():
        return None
    return float(m_b.group(1))


def round_bytes(cfg, lens0, width0, acc_hist):
    """Algorithmic bytes of each round's verify and realign launch.

    verify: B*(D+1)*V logits + drafts + outputs.
    realign: per row, its old content and its n = a+1 committed entries are read
    and S' positions (pad + content) are written, for every (layer, K|V, head):
    P * (sum(c) + sum(n) + B*S') with P the KV bytes of one position across
    layers, K and V and heads; plus tokens read, and tokens, position ids and mask
    written over [0, S')."""
    import numpy as np
    B, D, V = cfg.B, cfg.D, cfg.V
    es_logit = 4 if cfg.logit_dtype == 0 else 2
    P = cfg.kv_pos_bytes
    lens = lens0.astype(np.int64).copy()
    verify, realign = [], []
    for acc in acc_hist:
        n = acc.astype(np.int64) + 1
        snew = int((lens + n).max())
        kv = P * (int(lens.sum()) + int(n.sum()) + B * snew)
        meta = 4 * int(lens.sum()) + 4 * int(acc.sum()) + 12 * B + B * snew * 9 + 4 * B + 4
        realign.append(kv + meta)
        verify.append(B * (D + 1) * V * es_logit + B * D * 4 + 8 * B)
        lens = lens + n
    return np.array(verify, dtype=np.float64), np.array(realign, dtype=np.float64)


def cpu_baseline(cfg, plans, lens0, width0, tok0, mask0, rounds, layers):
    """The oracle (single-threaded C), as it stands, on the first `rounds` rounds
    of the same chain: verification of every row, realignment of `layers` of the
    cfg.L layers (layers are independent and identical work), scaled to all."""
    import numpy as np
    import oracle
    import synth
    layers = min(layers, cfg.L)
    lens, S, tok, mask = lens0.copy(), width0, tok0.copy(), mask0.copy()
    state = synth.kv_host(cfg, lens, S, True, layer0=0, nlayers=layers)
    spare = np.empty_like(state)
    t_ver = t_re = 0.0
    for r in range(rounds):
        plant, _, draft = plans[r]
        logits = synth.logits_host(cfg, r, plant)
        kvn = synth.kvnew_host(cfg, r, layer0=0, nlayers=layers)
        t0 = time.perf_counter()
        acc, nxt, _ = oracle.verify_greedy(logits, draft, cfg.B, cfg.D, cfg.V)
        t1 = time.perf_counter()
        out = oracle.realign_eqspec(state, kvn, lens, S, tok, mask, acc, nxt, draft, kv_out=spare)
        t2 = time.perf_counter()
        t_ver += t1 - t0
        t_re += t2 - t1
        spare, state = state, out["kv"]
        lens, S, tok, mask = out["len"], out["width"], out["tokens"], out["mask"]
    per_round = (t_ver + t_re * cfg.L / layers) / rounds
    return {
        "value": 1.0 / per_round,
        "unit": "rounds/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "rounds 0-%d of the same chain: greedy verify of all %d rows (%.1f ms/round) and EQSPEC realign "
                  "of layers 0-%d of %d (%.1f ms/round), realign time scaled by %d/%d; single-threaded C oracle; "
                  "%.1f s of CPU work" % (rounds - 1, cfg.B * cfg.D1, 1e3 * t_ver / rounds, layers - 1, cfg.L,
                                         1e3 * t_re / rounds, cfg.L, layers, t_ver + t_re),
        "host_cpus": os.cpu_count(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import synth.device as sdev
    import ragged_kv_realignment_amd as sd

    cfg = synth.CONFIGS[args.config]
    K, W = args.steps, args.warmup
    R = max(K, W, 1)
    cap = max(cfg.cap, cfg.len_hi + R * cfg.D1)
    kv_dt = sdev.TORCH_DT[cfg.kv_dtype]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    w = sdev.GreedyRounds(cfg, R)
    bufs = [sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cap, cfg.Dh, kv_dt) for _ in range(2)]
    ws = sd.workspace(cfg.B, cfg.D)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    acc_hist = torch.zeros((R, cfg.B), dtype=torch.int32, device=dev)
    nxt_hist = torch.zeros((R, cfg.B), dtype=torch.int32, device=dev)

    def run(n, ev=None):
        for r in range(n):
            src, dst = bufs[r % 2], bufs[(r + 1) % 2]
            if ev:
                ev[r][0].record()
            sd.verify_greedy(w.logits[r], w.drafts[r], ws=ws, status=status, accept_len=acc_hist[r],
                             next_token=nxt_hist[r])
            if ev:
                ev[r][1].record()
            sd.realign_eqspec(src, dst, w.kv_new[r], w.drafts[r], acc_hist[r], nxt_hist[r], status=status)
            if ev:
                ev[r][2].record()

    w.load_initial(bufs[0])
    torch.cuda.synchronize()
    run(W)
    torch.cuda.synchronize()
    w.load_initial(bufs[0])
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    run(K, ev)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    if int(status.item()) != 0:
        raise RuntimeError("device status %d during the timed rounds" % int(status.item()))
    ver_ms = np.array([ev[r][0].elapsed_time(ev[r][1]) for r in range(K)])
    re_ms = np.array([ev[r][1].elapsed_time(ev[r][2]) for r in range(K)])
    accs = acc_hist[:K].cpu().numpy()
    vbytes, rbytes = round_bytes(cfg, w.lens0, w.width0, accs)

    re_gbs = rbytes.sum() / (re_ms.sum() * 1e-3) / 1e9
    ve_gbs = vbytes.sum() / (ver_ms.sum() * 1e-3) / 1e9
    traffic = traffic_per_launch()

    copy_note = None
    if args.copy_calib_gib > 0:
        # a plain streaming elementwise kernel of known traffic (reads n bytes,
        # writes n bytes), used to scale the hardware byte counters
        n = int(args.copy_calib_gib * (1 << 30)) // 4 * 4
        a = torch.ones(n // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            torch.neg(a, out=b)
        c1.record()
        torch.cuda.synchronize()
        copy_note = {"kernel": "torch.neg float32", "read_bytes": n, "write_bytes": n,
                     "copy_gbs": 5 * 2 * n / (c0.elapsed_time(c1) * 1e-3) / 1e9}
        del a, b

    cpu = None
    if not args.no_cpu:
        del bufs
        torch.cuda.empty_cache()
        cpu = cpu_baseline(cfg, w.plans, w.lens0, w.width0, w.tok0, w.mask0, min(args.cpu_rounds, R),
                           args.cpu_layers)

    rounds_per_s = K / (total_ms * 1e-3)
    line = {
        "metric": METRIC,
        "value": rounds_per_s,
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": total_ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "%s: B=%d, D=%d, V=%d %s logits, KV %dx%dx%d %s, lengths U[%d,%d] left-padded, %d chained "
                        "greedy verify+EQSPEC rounds" % (cfg.name, cfg.B, cfg.D, cfg.V,
                                                         synth.DTYPE_NAME[cfg.logit_dtype], cfg.L, cfg.H, cfg.Dh,
                                                         synth.DTYPE_NAME[cfg.kv_dtype], cfg.len_lo, cfg.len_hi, K),
            "B": cfg.B, "D": cfg.D, "V": cfg.V, "layers": cfg.L, "kv_heads": cfg.H, "head_dim": cfg.Dh,
            "cap": cap, "global_batch": cfg.B,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_realign_eqspec",
            "achieved": re_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": re_gbs / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": float(rbytes.mean()),
            "avg_launch_us": float(re_ms.mean() * 1e3),
        },
        "verify": {
            "kernel": "k_verify_greedy",
            "achieved_gbs": ve_gbs,
            "frac": ve_gbs / PEAK_HBM_GBS,
            "algorithmic_bytes_per_launch": float(vbytes.mean()),
            "avg_launch_us": float(ver_ms.mean() * 1e3),
        },
        "realign_share_of_round": float(re_ms.sum() / total_ms),
        "cpu_baseline": cpu,
    }
    if copy_note:
        line["copy_calibration"] = copy_note
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
