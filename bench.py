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

The headline realigns in place: one rectangle, where only the bytes that
change move.  The out-of-place realignment (two rectangles, the full new one
written) is timed on the same rounds and reported beside it; both give the
same result.

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
_CSRC = os.path.join(ROOT, "ragged_kv_realignment_amd", "csrc")
_HEADERS = ("buffer_io.h", "device_common.h", "realign_params.h")
KERNEL = {False: "k_realign_eqspec", True: "k_realign_inplace"}
PAGE = 16  # positions per page of the paged-cache leg
SPIN_CYCLES_PER_LAUNCH = 200000  # GPU spin ahead of a pass, per launch queued behind it (~100 us at 2 GHz)
# counter summary and the sources of the realign kernel it was taken on, per realign mode
VERIFY_SOURCES = ("verify.hip", "coherent.h", "device_common.h", "launch.h", "wave_dpp.h")
SAMPLE_LOGITS_SOURCES = ("sample_logits.hip", "device_common.h", "launch.h", "wave_dpp.h")
TRAFFIC = {
    False: (os.path.join(ROOT, "profiles", "realign_eqspec_8b_gqa_traffic.txt"), ("realign.hip",) + _HEADERS),
    True: (os.path.join(ROOT, "profiles", "realign_inplace_8b_gqa_traffic.txt"),
           ("realign_inplace.hip",) + _HEADERS),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed rounds (default: the workload's round count)")
    ap.add_argument("--warmup", type=int, default=8, help="untimed rounds before the timed ones")
    ap.add_argument("--config", default="8b-gqa",
                    help="8b-gqa (default: the B=16 chain the metric is quoted on), 7b-mha, stoch or exspec")
    ap.add_argument("--cpu-rounds", type=int, default=64, help="oracle sample: rounds")
    ap.add_argument("--cpu-layers", type=int, default=36, help="oracle sample: KV layers realigned (scaled to all)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--trials", type=int, default=5,
                    help="uninstrumented timed passes over the K rounds (median reported)")
    ap.add_argument("--realign", choices=("all", "both", "inplace", "eqspec", "paged"), default="all",
                    help="chain workloads: realign in place on one buffer, out of place between two, on a paged "
                         "cache, in place and out of place (both), or all three; the headline is the first")
    ap.add_argument("--lifecycle", action="store_true",
                    help="exspec: pool rounds with sequences finishing and queued prompts admitted")
    ap.add_argument("--copy-calib-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration for profiling)")
    return ap.parse_args()


def source_sha(names):
    """First 16 hex digits of the SHA-256 of kernel sources under csrc/."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def realign_kernel_sha(inplace=False):
    return source_sha(TRAFFIC[inplace][1])


def _counter_ratio(path, sha_key, ratio_key, sources):
    """(traffic / algorithmic ratio, how) from a committed counter summary, or
    None when it is missing or was taken on other kernel sources."""
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_sha = re.search(r"^%s:\s*(\w+)" % sha_key, txt, re.M)
    m_r = re.search(r"^%s:\s*([0-9.eE+]+)" % ratio_key, txt, re.M)
    if not m_sha or not m_r or m_sha.group(1) != source_sha(sources):
        return None
    return float(m_r.group(1)), "rocprofv3 FETCH_SIZE + WRITE_SIZE over algorithmic bytes = %s (%s, taken over the " \
        "64-round chain on kernel sources %s), applied to this run's algorithmic bytes per launch" % (
            m_r.group(1), os.path.relpath(path, ROOT), m_sha.group(1))


def traffic_ratio(inplace=False):
    return _counter_ratio(TRAFFIC[inplace][0], "kernel_source_sha256_16", "traffic_over_algorithmic",
                          TRAFFIC[inplace][1])


def verify_sample_traffic(alg_bytes):
    r = _counter_ratio(os.path.join(ROOT, "profiles", "verify_sample_stoch_traffic.txt"),
                       "verify_sample_source_sha256_16", "verify_sample_traffic_over_algorithmic", VERIFY_SOURCES)
    return None if r is None else (r[0] * alg_bytes, r[1].replace("64-round chain", "stoch round"))


def sample_logits_traffic(alg_bytes):
    r = _counter_ratio(os.path.join(ROOT, "profiles", "verify_sample_stoch_traffic.txt"),
                       "sample_logits_source_sha256_16", "sample_logits_traffic_over_algorithmic",
                       SAMPLE_LOGITS_SOURCES)
    if r is None:
        return None
    return {"bytes_per_call": r[0] * alg_bytes,
            "how": r[1].replace("64-round chain", "stoch logits (statistics, mass and draw at top_p 1)")
                       .replace("per launch", "per call")}


def verify_traffic(alg_bytes):
    r = _counter_ratio(TRAFFIC[True][0], "verify_source_sha256_16", "verify_traffic_over_algorithmic",
                       VERIFY_SOURCES)
    return None if r is None else {"bytes_per_launch": r[0] * alg_bytes, "how": r[1]}


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


def round_bytes_inplace(cfg, lens0, width0, acc_hist):
    """Algorithmic bytes of each round's in-place realignment.

    Row b moves by shift = S' - S - n_b positions.  A row with content that
    moves reads and writes its c_b positions; a move to higher positions also
    writes `shift` positions of zero pad; every row reads and writes its n_b
    committed entries.  Token ids move with the content; pad and committed
    token ids, and position ids and mask over [0, S'), are written."""
    import numpy as np
    B = cfg.B
    P = cfg.kv_pos_bytes
    lens = lens0.astype(np.int64).copy()
    S = int(width0)
    out = []
    for acc in acc_hist:
        n = acc.astype(np.int64) + 1
        snew = int((lens + n).max())
        shift = snew - S - n
        moved = (shift != 0) & (lens > 0)
        kv = P * (2 * int(lens[moved].sum()) + int(np.maximum(shift, 0).sum()) + 2 * int(n.sum()))
        pout = snew - lens - n
        meta = (8 * int(lens[moved].sum()) + 4 * int(pout.sum()) + 4 * int(n.sum()) + 5 * B * snew +
                4 * int(acc.sum()) + 16 * B + 8)
        out.append(kv + meta)
        lens, S = lens + n, snew
    return np.array(out, dtype=np.float64)


def round_bytes_paged(cfg, lens0, acc_hist, page):
    """Algorithmic bytes of each round's realignment on a paged cache: every
    row's n_b committed entries are read from the speculative KV and written to
    their page slots; token ids of the old content are read and the rectangle
    view (token ids, position ids, mask over [0, S')) written; committed token
    ids, lengths and new block-table entries written."""
    import numpy as np
    B = cfg.B
    P = cfg.kv_pos_bytes
    lens = lens0.astype(np.int64).copy()
    out = []
    for acc in acc_hist:
        n = acc.astype(np.int64) + 1
        snew = int((lens + n).max())
        new_blocks = int(((lens + n + page - 1) // page - (lens + page - 1) // page).sum())
        kv = 2 * P * int(n.sum())
        meta = (9 * B * snew + 4 * int(lens.sum()) + 4 * int(n.sum()) + 4 * int(acc.sum()) + 16 * B +
                4 * new_blocks + 8)
        out.append(kv + meta)
        lens = lens + n
    return np.array(out, dtype=np.float64)


def _oracle_chain(cfg, plans, lens0, width0, tok0, mask0, rounds, layers):
    """Seconds the oracle spends on greedy verification and on the EQSPEC
    realignment of `layers` layers over the first `rounds` rounds of the chain."""
    import numpy as np
    import oracle
    import synth
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
    return t_ver, t_re


def cpu_baseline(cfg, plans, lens0, width0, tok0, mask0, rounds, layers):
    """The oracle (C), as it stands, on the first `rounds` rounds of the same
    chain: verification of every row, realignment of `layers` of the cfg.L
    layers (layers are independent and identical work), scaled to all.  The
    reported value is the single-threaded build; the same sample run through
    the OpenMP build of the same source (rows and KV segments over all host
    threads) is reported beside it under "all_cores"."""
    import oracle
    layers = min(layers, cfg.L)

    def rate(t_ver, t_re):
        return rounds / (t_ver + t_re * cfg.L / layers)

    t_ver, t_re = _oracle_chain(cfg, plans, lens0, width0, tok0, mask0, rounds, layers)
    oracle.use_threads(True)
    try:
        threads = oracle.threads()
        m_ver, m_re = _oracle_chain(cfg, plans, lens0, width0, tok0, mask0, rounds, layers)
    finally:
        oracle.use_threads(False)
    return {
        "value": rate(t_ver, t_re),
        "unit": "rounds/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "rounds 0-%d of the same chain: greedy verify of all %d rows (%.1f ms/round) and EQSPEC realign "
                  "of layers 0-%d of %d (%.1f ms/round), realign time scaled by %d/%d; single-threaded C oracle; "
                  "%.1f s of CPU work" % (rounds - 1, cfg.B * cfg.D1, 1e3 * t_ver / rounds, layers - 1, cfg.L,
                                         1e3 * t_re / rounds, cfg.L, layers, t_ver + t_re),
        "host_cpus": os.cpu_count(),
        "all_cores": {"value": rate(m_ver, m_re), "unit": "rounds/s", "cores": threads, "kind": "oracle (OpenMP build)",
                      "sample": "the same sample on %d threads: verify %.1f ms/round, realign %.1f ms/round "
                                "(before scaling), %.1f s wall" % (threads, 1e3 * m_ver / rounds,
                                                                   1e3 * m_re / rounds, m_ver + m_re)},
    }


def _events(n, k):
    import torch
    return [[torch.cuda.Event(enable_timing=True) for _ in range(k)] for _ in range(n)]


def _ms(ev, i, j):
    import numpy as np
    return np.array([e[i].elapsed_time(e[j]) for e in ev])


def copy_calibration(gib, dev):
    """A plain streaming elementwise kernel of known traffic (reads n bytes, writes
    n bytes), used to scale the hardware byte counters."""
    import torch
    n = int(gib * (1 << 30)) // 4 * 4
    a = torch.ones(n // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        torch.neg(a, out=b)
    c1.record()
    torch.cuda.synchronize()
    return {"kernel": "torch.neg float32", "read_bytes": n, "write_bytes": n,
            "copy_gbs": 5 * 2 * n / (c0.elapsed_time(c1) * 1e-3) / 1e9}


def practical_ceiling(dev, gib=2.0):
    """Streaming rates of plain torch elementwise kernels on the same GPU: an
    elementwise op that reads n and writes n bytes (torch.neg), and a fill that
    writes n bytes.  They bound what a copy-shaped kernel reaches in practice."""
    import torch
    n = int(gib * (1 << 30)) // 4 * 4
    a = torch.ones(n // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)

    def rate(fn, nbytes, reps=5):
        fn()
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(reps):
            fn()
        c1.record()
        torch.cuda.synchronize()
        return reps * nbytes / (c0.elapsed_time(c1) * 1e-3) / 1e9

    out = {"read_write_gbs": rate(lambda: torch.neg(a, out=b), 2 * n), "write_gbs": rate(lambda: b.fill_(2.0), n),
           "kernels": "torch.neg (reads n, writes n) and fill_ (writes n) on %d-byte float32 buffers" % n}
    del a, b
    torch.cuda.empty_cache()
    return out


def _line(metric, value, K, W, ms_per_step, dtype, config, roofline, cpu, extra):
    line = {"metric": metric, "value": value, "unit": "rounds/s", "n_gpus": 1, "steps": K, "warmup": W,
            "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype, "data": "synthetic", "config": config, "roofline": roofline}
    line.update(extra)
    line["cpu_baseline"] = cpu
    return line


def _roof(kernel, gbs, bytes_per_launch, us, traffic=None):
    return {"bound": "hbm", "kernel": kernel, "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": bytes_per_launch,
            "avg_launch_us": us}


def _time_chain(args, cfg, w, mode, K, W, cap):
    """Times K chained rounds (after W untimed ones and a reset of the initial
    state) with the realignment done in place on one buffer ("inplace"), out of
    place between two ("eqspec"), or on a paged cache ("paged", also replayed
    from a HIP graph).  Rounds/s from uninstrumented passes; per-launch
    durations from one more pass with HIP events on the launch stream."""
    import numpy as np
    import torch
    import synth.device as sdev
    import ragged_kv_realignment_amd as sd

    R = max(K, W, 1)
    dev = torch.device("cuda", 0)
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    bufs = [sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cap, cfg.Dh, tdt) for _ in range(1 if mode != "eqspec" else 2)]
    if mode == "paged":
        mb = -(-cap // PAGE)
        cache = sd.PagedKV.empty(cfg.L, cfg.B, cfg.H, cfg.Dh, cfg.B * mb, PAGE, mb, tdt)
        width = torch.zeros(1, dtype=torch.int32, device=dev)
        view = (torch.zeros((cfg.B, cap), dtype=torch.int32, device=dev),
                torch.zeros((cfg.B, cap), dtype=torch.int32, device=dev),
                torch.zeros((cfg.B, cap), dtype=torch.int8, device=dev))
        every_row = torch.arange(cfg.B, dtype=torch.int32, device=dev)
    ws = sd.workspace(cfg.B, cfg.D)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    acc_hist = torch.zeros((R, cfg.B), dtype=torch.int32, device=dev)
    nxt_hist = torch.zeros((R, cfg.B), dtype=torch.int32, device=dev)

    def run(n, ev=None):
        for r in range(n):
            if ev:
                ev[r][0].record()
            sd.verify_greedy(w.logits[r], w.drafts[r], ws=ws, status=status, accept_len=acc_hist[r],
                             next_token=nxt_hist[r])
            if ev:
                ev[r][1].record()
            if mode == "paged":
                sd.paged_append(cache, w.kv_new[r], w.drafts[r], acc_hist[r], nxt_hist[r], width=width,
                                rect_tokens=view[0], rect_pos=view[1], rect_mask=view[2], status=status)
            elif mode == "inplace":
                sd.realign_eqspec_inplace(bufs[0], w.kv_new[r], w.drafts[r], acc_hist[r], nxt_hist[r],
                                          status=status)
            else:
                sd.realign_eqspec(bufs[r % 2], bufs[(r + 1) % 2], w.kv_new[r], w.drafts[r], acc_hist[r],
                                  nxt_hist[r], status=status)
            if ev:
                ev[r][2].record()

    def reset():
        w.load_initial(bufs[0])
        if mode == "paged":
            sd.paged_retire(cache, every_row, status=status)
            sd.paged_admit(cache, bufs[0], status=status)
        torch.cuda.synchronize()

    reset()
    run(W)
    torch.cuda.synchronize()
    # rounds/s: the median of `trials` uninstrumented passes over the same K
    # rounds, each from the initial state (events only around the pass)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    trials, acc0 = [], None
    for _ in range(max(1, args.trials)):
        reset()
        start.record()
        run(K)
        end.record()
        torch.cuda.synchronize()
        trials.append(start.elapsed_time(end))
        if int(status.item()) != 0:
            raise RuntimeError("device status %d during the timed rounds (%s)" % (int(status.item()), mode))
        acc = acc_hist[:K].cpu().numpy()
        if acc0 is not None and not np.array_equal(acc, acc0):
            raise RuntimeError("passes over the same rounds disagree (%s)" % mode)
        acc0 = acc
    # per-launch durations: one more pass with events around every launch
    reset()
    ev = _events(K, 3)
    start.record()
    run(K, ev)
    end.record()
    torch.cuda.synchronize()
    if int(status.item()) != 0 or not np.array_equal(acc_hist[:K].cpu().numpy(), acc0):
        raise RuntimeError("the instrumented pass differs (%s)" % mode)
    out = {"total_ms": float(np.median(trials)), "trials_ms": trials, "instrumented_ms": start.elapsed_time(end),
           "ver_ms": _ms(ev, 0, 1), "re_ms": _ms(ev, 1, 2), "acc": acc0}
    if mode == "paged":
        # the same K rounds captured once in a HIP graph and replayed from the
        # initial state: no host work per round; the replay must reproduce the
        # eager rounds exactly
        want_len, want_tok = cache.len.clone(), cache.tokens.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(K)
        reset()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        g.replay()
        g1.record()
        torch.cuda.synchronize()
        if not (np.array_equal(acc_hist[:K].cpu().numpy(), out["acc"]) and torch.equal(cache.len, want_len) and
                torch.equal(cache.tokens, want_tok)):
            raise RuntimeError("the graph replay differs from the eager rounds")
        out["graph_ms"] = g0.elapsed_time(g1)
        del g
        del cache
    del bufs
    torch.cuda.empty_cache()
    return out


def cycle_stats(acc, D, rounds_per_s=None):
    """Per-cycle measurements of verification: where the first rejection fell
    (accept length a = the position of the first rejected draft; a = D means
    none was rejected), drafts accepted and tokens committed (a + 1) per round,
    and the committed-token rate at the measured round rate."""
    import numpy as np
    acc = np.asarray(acc, dtype=np.int64)
    hist = np.bincount(acc.reshape(-1), minlength=D + 1)[:D + 1]
    per_round = (acc + 1).sum(axis=1)
    out = {"accept_len_histogram": hist.tolist(),
           "first_rejection_position_histogram": hist[:D].tolist(),
           "no_rejection_rows": int(hist[D]),
           "accepted_drafts_per_round": float(acc.sum(axis=1).mean()),
           "committed_tokens_per_round": float(per_round.mean()),
           "committed_tokens_per_row_round": float((acc + 1).mean()),
           "committed_tokens_per_round_min_max": [int(per_round.min()), int(per_round.max())]}
    if rounds_per_s:
        out["committed_tokens_per_s"] = float(per_round.mean() * rounds_per_s)
    return out


def host_info():
    """The host the benchmark ran on: logical CPUs, CPUs this process may use, RAM."""
    ram = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    ram = int(line.split()[1]) * 1024
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu_count": os.cpu_count(), "cpus_usable": aff, "ram_bytes": ram}


def device_memory(dev, kv_bytes=None, kv_content_bytes=None):
    import torch
    out = {"peak_allocated_bytes": int(torch.cuda.max_memory_allocated(dev)),
           "device_total_bytes": int(torch.cuda.get_device_properties(dev).total_memory)}
    if kv_bytes is not None:
        out["kv_cache_bytes"] = int(kv_bytes)
    if kv_content_bytes is not None:
        out["kv_content_bytes_final"] = int(kv_content_bytes)
    return out


def _measure_lib():
    import ctypes as C
    L = C.CDLL(os.path.join(ROOT, "ragged_kv_realignment_amd", "libspecdec_measure.so"))
    L.specdec_measure_read_floor.argtypes = [C.c_void_p, C.c_int, C.c_int64, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                             C.c_int, C.c_void_p]
    L.specdec_measure_read_floor.restype = C.c_int
    L.specdec_measure_stats_floor.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                              C.c_int, C.c_void_p]
    L.specdec_measure_stats_floor.restype = C.c_int
    return L


def verify_alone(cfg, w, K):
    """Greedy verification over the K rounds' logits with nothing between the
    launches, beside two references on the same cold buffers: a bare read with
    verification's exact launch shape and loads (its floor), and torch.argmax
    (a library doing the same arithmetic).  Each is timed twice: HIP events
    around every launch, and events around the whole pass of K launches (the
    pass average carries no per-launch event, but the gaps between launches)."""
    import numpy as np
    import torch
    import ragged_kv_realignment_amd as sd

    dev = torch.device("cuda", 0)
    ws = sd.workspace(cfg.B, cfg.D)
    acc = torch.zeros((K, cfg.B), dtype=torch.int32, device=dev)
    nxt = torch.zeros((K, cfg.B), dtype=torch.int32, device=dev)
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    M = _measure_lib()
    es = 4 if cfg.logit_dtype == 0 else 2
    stream = torch.cuda.current_stream().cuda_stream

    def floor(r):
        g = M.specdec_measure_read_floor(w.logits[r].data_ptr(), es, cfg.V, cfg.B, cfg.D, cfg.V, sink.data_ptr(),
                                         sink.numel(), stream)
        if g < 0:
            raise RuntimeError("bare-read launch failed")

    kernels = {
        "verify": lambda r: sd.verify_greedy(w.logits[r], w.drafts[r], ws=ws, accept_len=acc[r], next_token=nxt[r]),
        "floor": floor,
        "torch_argmax": lambda r: torch.argmax(w.logits[r], dim=-1),
    }
    out = {}
    for name, fn in kernels.items():
        fn(0)
        torch.cuda.synchronize()
        # each pass starts behind a spin kernel long enough for the host to
        # queue all K launches, so the pass runs at the GPU's pace rather than
        # the host's (the binding's checks take longer than a launch runs)
        ev = _events(K, 2)
        torch.cuda._sleep(SPIN_CYCLES_PER_LAUNCH * K)
        for r in range(K):
            ev[r][0].record()
            fn(r)
            ev[r][1].record()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SPIN_CYCLES_PER_LAUNCH * K)
        a.record()
        for r in range(K):
            fn(r)
        b.record()
        torch.cuda.synchronize()
        out[name] = {"avg_launch_us": float(_ms(ev, 0, 1).mean() * 1e3), "pass_avg_us": a.elapsed_time(b) * 1e3 / K}
    return out


def bench_chain(args, cfg):
    """Chained greedy verify + EQSPEC rounds of a left-padded batch (8b-gqa, 7b-mha).

    The headline realigns in place (one buffer); with --realign both (the
    default) the out-of-place realignment is timed on the same rounds and
    reported beside it."""
    import torch
    import synth
    import synth.device as sdev

    K = args.steps if args.steps is not None else cfg.rounds
    W = args.warmup
    R = max(K, W, 1)
    cap = max(cfg.cap, cfg.len_hi + R * cfg.D1)
    dev = torch.device("cuda", 0)
    w = sdev.GreedyRounds(cfg, R)
    modes = {"all": ("inplace", "eqspec", "paged"), "both": ("inplace", "eqspec")}.get(args.realign, (args.realign,))
    runs = {m: _time_chain(args, cfg, w, m, K, W, cap) for m in modes}
    with_traffic = cfg.name == "8b-gqa"  # the workload the counters were taken on

    def roof(mode):
        r = runs[mode]
        if mode == "paged":
            pb = round_bytes_paged(cfg, w.lens0, r["acc"], PAGE)
            gbs = pb.sum() / (r["re_ms"].sum() * 1e-3) / 1e9
            return _roof("k_paged_append", gbs, float(pb.mean()),
                         float(r["re_ms"].mean() * 1e3))
        fn = round_bytes_inplace if mode == "inplace" else (lambda *a: round_bytes(*a)[1])
        rbytes = fn(cfg, w.lens0, w.width0, r["acc"])
        gbs = rbytes.sum() / (r["re_ms"].sum() * 1e-3) / 1e9
        tr = traffic_ratio(mode == "inplace") if with_traffic else None
        out = _roof(KERNEL[mode == "inplace"], gbs, float(rbytes.mean()), float(r["re_ms"].mean() * 1e3),
                    None if tr is None else tr[0] * float(rbytes.mean()))
        if tr is not None:
            out["traffic_how"] = tr[1]
        return out

    head = runs[modes[0]]
    vbytes, _ = round_bytes(cfg, w.lens0, w.width0, head["acc"])
    ve_gbs = vbytes.sum() / (head["ver_ms"].sum() * 1e-3) / 1e9
    alone = verify_alone(cfg, w, K)
    logit_bytes = cfg.B * cfg.D1 * cfg.V * (4 if cfg.logit_dtype == 0 else 2)
    extra = {}
    if args.copy_calib_gib > 0:
        extra["copy_calibration"] = copy_calibration(args.copy_calib_gib, dev)
    ceiling = practical_ceiling(dev)
    extra["practical_ceiling"] = ceiling
    extra.update({
        "verify": {"kernel": "k_verify_greedy", "achieved_gbs": ve_gbs, "frac": ve_gbs / PEAK_HBM_GBS,
                   "algorithmic_bytes_per_launch": float(vbytes.mean()),
                   "avg_launch_us": float(head["ver_ms"].mean() * 1e3),
                   "traffic": verify_traffic(float(vbytes.mean())),
                   "alone": {**alone["verify"], "how": "the same %d launches with nothing between them" % K},
                   "practical_floor": {
                       **alone["floor"], "gbs": logit_bytes / (alone["floor"]["avg_launch_us"] * 1e-6) / 1e9,
                       "kernel": "bare read of the same cold logits with verification's grid, workgroups and "
                                 "16-byte loads, no reduction (libspecdec_measure.so)"},
                   "frac_of_practical": alone["floor"]["avg_launch_us"] / alone["verify"]["avg_launch_us"],
                   "frac_of_practical_pass": alone["floor"]["pass_avg_us"] / alone["verify"]["pass_avg_us"],
                   "torch_argmax": {**alone["torch_argmax"],
                                    "kernel": "torch.argmax(logits, -1) over the same buffers (first maximum)"}},
        "realign_share_of_round": float(head["re_ms"].sum() / head["instrumented_ms"]),
        "timing": {"trials_ms": head["trials_ms"], "instrumented_pass_ms": head["instrumented_ms"],
                   "how": "value and ms_per_step: median of the uninstrumented passes; per-kernel figures: one more "
                          "pass with HIP events around every launch on the launch stream"},
    })
    if "eqspec" in modes and modes[0] != "eqspec":
        o = runs["eqspec"]
        extra["out_of_place"] = {"value": K / (o["total_ms"] * 1e-3), "unit": "rounds/s",
                                 "ms_per_step": o["total_ms"] / K, "roofline": roof("eqspec")}
    if "paged" in modes and modes[0] != "paged":
        o = runs["paged"]
        pb = round_bytes_paged(cfg, w.lens0, o["acc"], PAGE)
        gbs = pb.sum() / (o["re_ms"].sum() * 1e-3) / 1e9
        extra["paged"] = {"value": K / (o["total_ms"] * 1e-3), "unit": "rounds/s", "ms_per_step": o["total_ms"] / K,
                          "graph": {"value": K / (o["graph_ms"] * 1e-3), "unit": "rounds/s",
                                    "ms_per_step": o["graph_ms"] / K,
                                    "how": "the same %d rounds captured in one HIP graph, replayed once" % K},
                          "page_positions": PAGE,
                          "call": "specdec_verify_greedy, then specdec_paged_append",
                          "realign": {"kernels": "k_paged_append",
                                      "achieved_gbs": gbs, "frac": gbs / PEAK_HBM_GBS,
                                      "algorithmic_bytes_per_call": float(pb.mean()),
                                      "avg_call_us": float(o["re_ms"].mean() * 1e3)}}
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, w.plans, w.lens0, w.width0, w.tok0, w.mask0, min(args.cpu_rounds, R),
                           args.cpu_layers)
    how = {"inplace": " (realigned in place)", "eqspec": " (realigned out of place)",
           "paged": " (paged cache, realigned as metadata)"}[modes[0]]
    workload = "%s: B=%d, D=%d, V=%d %s logits, KV %dx%dx%d %s, lengths U[%d,%d] left-padded, %d chained " \
               "greedy verify+EQSPEC rounds%s" % (
                   cfg.name, cfg.B, cfg.D, cfg.V, synth.DTYPE_NAME[cfg.logit_dtype], cfg.L, cfg.H, cfg.Dh,
                   synth.DTYPE_NAME[cfg.kv_dtype], cfg.len_lo, cfg.len_hi, K, how)
    config = {
        "workload": workload,
        "B": cfg.B, "D": cfg.D, "V": cfg.V, "layers": cfg.L, "kv_heads": cfg.H, "head_dim": cfg.Dh, "cap": cap,
        "global_batch": cfg.B,
    }
    metric = METRIC if cfg.name == "8b-gqa" else METRIC.replace("at B=16", "at B=%d (%s)" % (cfg.B, cfg.name))
    rps = K / (head["total_ms"] * 1e-3)
    final_lens = w.lens0.astype("int64") + (head["acc"].astype("int64") + 1).sum(axis=0)
    extra["cycle"] = cycle_stats(head["acc"], cfg.D, rps)
    extra["memory"] = device_memory(dev, kv_bytes=cfg.L * 2 * cfg.B * cfg.H * cap * cfg.Dh * (
        4 if cfg.kv_dtype == 0 else 2), kv_content_bytes=cfg.kv_pos_bytes * int(final_lens.sum()))
    extra["host"] = host_info()
    headroof = roof(modes[0])
    if modes[0] in ("inplace", "eqspec"):  # a copy-shaped kernel: its rate against the measured streaming rate
        headroof["frac_of_practical"] = headroof["achieved"] / ceiling["read_write_gbs"]
    return _line(metric, K / (head["total_ms"] * 1e-3), K, W, head["total_ms"] / K, synth.DTYPE_NAME[cfg.kv_dtype],
                 config, headroof, cpu, extra)


def _time_sample_logits(cfg, K):
    """Sampled verification from the workload's raw fp32 logits (temperature
    0.8, with and without a top-p 0.9 nucleus), K calls each, timed two ways
    with events on the launch stream: cold, each call after a 512 MiB fill that
    evicts the logits from the 256 MB Infinity Cache (they come from HBM), and
    warm, K calls queued back to back behind a spin kernel (the 69.6 MB of
    logits stay in the Infinity Cache).  Algorithmic bytes: one read of every
    target and draft logit.  Beside them, the same two timings of a bare read
    of the same logits with the statistics kernel's launch (its floor); the
    top_p 1 call reports its fraction of that floor."""
    import torch
    import synth
    import ragged_kv_realignment_amd as sd

    dev = torch.device("cuda", 0)
    tl, dl, draft, u_acc, u_draw = synth.sampled_logits_round(cfg, 0)
    t, d, dd, dua, dud = (torch.from_numpy(x).to(dev) for x in (tl, dl, draft, u_acc, u_draw))
    ws = sd.sample_workspace(cfg.B, cfg.D, cfg.V, dev)
    acc = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    nxt = torch.zeros_like(acc)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    nbytes = float(tl.nbytes + dl.nbytes)
    out = {"logits": "target [%d][%d][%d] and draft [%d][%d][%d] fp32" % (cfg.B, cfg.D1, cfg.V, cfg.B, cfg.D, cfg.V),
           "algorithmic_bytes_per_call": nbytes}
    M = _measure_lib()
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def floor_read():
        if M.specdec_measure_stats_floor(t.data_ptr(), d.data_ptr(), 4, cfg.B, cfg.D, cfg.V, sink.data_ptr(),
                                         sink.numel(), stream) < 0:
            raise RuntimeError("bare-read launch failed")

    for top_p in (1.0, 0.9, "floor"):
        if top_p == "floor":
            call = floor_read
        else:
            def call(top_p=top_p):
                sd.verify_sample_logits(t, d, dd, dua, dud, cfg.temperature, top_p=top_p, ws=ws, accept_len=acc,
                                        next_token=nxt, status=status)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ev = _events(K, 2)
        for r in range(K):
            flush.fill_(r & 255)
            ev[r][0].record()
            call()
            ev[r][1].record()
        torch.cuda.synchronize()
        cold = _ms(ev, 0, 1).mean()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SPIN_CYCLES_PER_LAUNCH * 4 * K)
        a.record()
        for _ in range(K):
            call()
        b.record()
        torch.cuda.synchronize()
        warm = a.elapsed_time(b) / K
        entry = {"avg_call_us": float(cold * 1e3), "achieved_gbs": nbytes / (cold * 1e-3) / 1e9,
                 "how": "cold: after a 512 MiB fill, events around the call",
                 "warm": {"avg_call_us": float(warm * 1e3), "achieved_gbs": nbytes / (warm * 1e-3) / 1e9,
                          "how": "logits in the Infinity Cache: calls queued back to back"}}
        if top_p == "floor":
            entry["kernel"] = ("bare read of the same target and draft logits with the statistics kernel's grid, "
                               "workgroups and 16-byte non-temporal loads, no arithmetic (libspecdec_measure.so)")
            out["practical_floor"] = entry
            one = out["top_p=1"]
            one["frac_of_practical"] = entry["avg_call_us"] / one["avg_call_us"]
            one["warm"]["frac_of_practical"] = entry["warm"]["avg_call_us"] / one["warm"]["avg_call_us"]
        else:
            out["top_p=%g" % top_p] = entry
        if top_p == 1.0:
            out["top_p=1"]["traffic"] = sample_logits_traffic(nbytes)
    if int(status.item()) != 0:
        raise RuntimeError("device status %d in sampled verification from logits" % int(status.item()))
    return out


def bench_stoch(args, cfg):
    """Sampled verification + EQSPEC realign of the fp16 cache; the same out-of-place
    round is repeated from the same state."""
    import numpy as np
    import torch
    import oracle
    import synth
    import synth.device as sdev
    import ragged_kv_realignment_amd as sd

    K = args.steps if args.steps is not None else 16
    W = args.warmup
    dev = torch.device("cuda", 0)
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    lens = synth.lengths(cfg)
    S = int(lens.max())
    p, q, draft, u_acc, u_draw = synth.sampled_round(cfg, 0)
    src = sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, tdt)
    dst = sd.SeqBuf.empty(cfg.L, cfg.B, cfg.H, cfg.cap, cfg.Dh, tdt)
    sdev.fill_kv(cfg, src.kv, torch.from_numpy(lens).to(dev), S, True)
    tok, pos, mask = synth.tokens_host(cfg, lens, S, True)
    src.tokens.copy_(torch.from_numpy(tok))
    src.pos.copy_(torch.from_numpy(pos))
    src.mask.copy_(torch.from_numpy(mask))
    src.len.copy_(torch.from_numpy(lens))
    src.width.fill_(S)
    kv_new = torch.empty((cfg.L, 2, cfg.B, cfg.H, cfg.D1, cfg.Dh), dtype=tdt, device=dev)
    sdev.fill_kvnew(cfg, 0, kv_new)
    dp, dq, dd, dua, dud = (torch.from_numpy(x).to(dev) for x in (p, q, draft, u_acc, u_draw))
    acc = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    nxt = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sws = sd.sample_verify_workspace(cfg.B, cfg.D, cfg.V)

    def run(n, ev=None):
        for r in range(n):
            if ev:
                ev[r][0].record()
            sd.verify_sample(dp, dq, dd, dua, dud, status=status, accept_len=acc, next_token=nxt, ws=sws)
            if ev:
                ev[r][1].record()
            sd.realign_eqspec(src, dst, kv_new, dd, acc, nxt, status=status)
            if ev:
                ev[r][2].record()

    run(W)
    torch.cuda.synchronize()
    ev = _events(K, 3)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    run(K, ev)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    if int(status.item()) != 0:
        raise RuntimeError("device status %d during the timed rounds" % int(status.item()))
    ver_ms, re_ms = _ms(ev, 0, 1), _ms(ev, 1, 2)
    a = acc.cpu().numpy()
    # sampled verify reads the accepted drafts' p(x), q(x) and one residual (p, q rows) or bonus (p row)
    vbytes = float(sum(16 * min(int(x) + 1, cfg.D) + (8 if x < cfg.D else 4) * cfg.V + 12 for x in a))
    _, rb = round_bytes(cfg, lens, S, a[None, :])
    rbytes = float(rb[0])
    re_gbs = rbytes / (re_ms.mean() * 1e-3) / 1e9
    ve_gbs = vbytes / (ver_ms.mean() * 1e-3) / 1e9
    # sampled verification alone: K launches queued behind a spin kernel, events
    # around the pass (no per-launch event, nothing between the launches)
    torch.cuda._sleep(SPIN_CYCLES_PER_LAUNCH * K)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(K):
        sd.verify_sample(dp, dq, dd, dua, dud, status=status, accept_len=acc, next_token=nxt, ws=sws)
    a1.record()
    torch.cuda.synchronize()
    ver_alone_us = a0.elapsed_time(a1) * 1e3 / K
    logits_legs = _time_sample_logits(cfg, K)
    cpu = None
    if not args.no_cpu:
        del src, dst
        torch.cuda.empty_cache()
        layers = min(args.cpu_layers, 2)
        kv_l = synth.kv_host(cfg, lens, S, True, layer0=0, nlayers=layers)
        kvn_l = synth.kvnew_host(cfg, 0, layer0=0, nlayers=layers)
        out = np.empty_like(kv_l)
        reps = 4

        def timed():
            t0 = time.perf_counter()
            for _ in range(reps):
                oacc, onxt, _ = oracle.verify_sample(p, q, draft, u_acc, u_draw)
            t1 = time.perf_counter()
            for _ in range(reps):
                oracle.realign_eqspec(kv_l, kvn_l, lens, S, tok, mask, oacc, onxt, draft, kv_out=out)
            t2 = time.perf_counter()
            return (t1 - t0) / reps, (t2 - t1) / reps

        t_ver, t_re = timed()
        oracle.use_threads(True)  # the OpenMP build: the realignment's KV segments over all threads
        try:
            threads = oracle.threads()
            m_ver, m_re = timed()
        finally:
            oracle.use_threads(False)
        cpu = {"value": 1.0 / (t_ver + t_re * cfg.L / layers), "unit": "rounds/s", "cores": 1, "kind": "oracle",
               "sample": "%d repeats of the round: sampled verify of all %d rows (%.1f ms) and EQSPEC realign of "
                         "layers 0-%d of %d (%.1f ms), realign scaled by %d/%d; single-threaded C oracle"
                         % (reps, cfg.B, 1e3 * t_ver, layers - 1, cfg.L, 1e3 * t_re, cfg.L, layers),
               "host_cpus": os.cpu_count(),
               "all_cores": {"value": 1.0 / (m_ver + m_re * cfg.L / layers), "unit": "rounds/s", "cores": threads,
                             "kind": "oracle (OpenMP build)",
                             "sample": "the same sample on %d threads (the sampled verify stays on one): verify "
                                       "%.1f ms, realign %.1f ms before scaling" % (threads, 1e3 * m_ver,
                                                                                   1e3 * m_re)}}
    config = {"workload": "stoch: B=%d, D=%d, V=%d fp32 p/q (softmax(l/0.8)), KV %dx%dx%d fp16, lengths U[%d,%d], "
                          "one sampled verify + EQSPEC round repeated" % (cfg.B, cfg.D, cfg.V, cfg.L, cfg.H, cfg.Dh,
                                                                         cfg.len_lo, cfg.len_hi),
              "B": cfg.B, "D": cfg.D, "V": cfg.V, "cap": cfg.cap, "global_batch": cfg.B}
    vt = verify_sample_traffic(vbytes)
    vroof = _roof("k_verify_sample", ve_gbs, vbytes, float(ver_ms.mean() * 1e3), None if vt is None else vt[0])
    if vt is not None:
        vroof["traffic_how"] = vt[1]
    vroof["alone"] = {"pass_avg_us": ver_alone_us, "gbs": vbytes / (ver_alone_us * 1e-6) / 1e9,
                      "frac": vbytes / (ver_alone_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                      "how": "%d launches queued behind a spin kernel, events around the pass (the same p and q "
                             "each time: the stop rows stay in the Infinity Cache)" % K}
    extra = {"verify": {"kernel": "k_verify_sample", "achieved_gbs": ve_gbs, "frac": ve_gbs / PEAK_HBM_GBS,
                        "algorithmic_bytes_per_launch": vbytes, "avg_launch_us": float(ver_ms.mean() * 1e3),
                        "roofline": vroof},
             "cycle": cycle_stats(a[None, :], cfg.D, K / (total_ms * 1e-3)),
             "memory": device_memory(dev),
             "host": host_info(),
             "verify_from_logits": logits_legs,
             "realign_share_of_round": float(re_ms.sum() / total_ms)}
    return _line("sampled verify+realign rounds/sec and realign HBM GB/s (stoch, B=32)", K / (total_ms * 1e-3), K, W,
                 total_ms / K, "f16", config,
                 _roof("k_realign_eqspec", re_gbs, rbytes, float(re_ms.mean() * 1e3)), cpu, extra)


def bench_exspec(args, cfg):
    """Pool rounds: group by length, gather mixed batches, verify every sequence,
    append committed entries in place."""
    import numpy as np
    import torch
    import oracle
    import synth
    import synth.device as sdev
    import ragged_kv_realignment_amd as sd

    K = args.steps if args.steps is not None else cfg.rounds
    W = 0  # rounds change the pool; the timed chain starts from the initial pool
    N, G = cfg.B, cfg.group
    dev = torch.device("cuda", 0)
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    cap = max(cfg.cap, cfg.len_hi + K * cfg.D1)
    lens0 = synth.lengths(cfg)
    pool = sd.SeqBuf.empty(cfg.L, N, cfg.H, cap, cfg.Dh, tdt, pool=True)
    sdev.fill_kv(cfg, pool.kv, torch.from_numpy(lens0).to(dev), 0, False)
    tok0, _, _ = synth.tokens_host(cfg, lens0, 0, False, cap=cap)
    pool.tokens.copy_(torch.from_numpy(tok0))
    pool.len.copy_(torch.from_numpy(lens0))
    ng = (N + G - 1) // G
    rect = sd.SeqBuf.empty(cfg.L, N, cfg.H, cap, cfg.Dh, tdt, groups=ng)
    plans = [synth.plan_greedy(cfg, r) for r in range(K)]
    logits = torch.empty((K, N, cfg.D1, cfg.V), dtype=sdev.TORCH_DT[cfg.logit_dtype], device=dev)
    keep = [sdev.fill_logits(cfg, r, plans[r][0], logits[r]) for r in range(K)]
    kv_new = torch.empty((K, cfg.L, 2, N, cfg.H, cfg.D1, cfg.Dh), dtype=tdt, device=dev)
    for r in range(K):
        sdev.fill_kvnew(cfg, r, kv_new[r])
    drafts = torch.from_numpy(np.stack([pl[2] for pl in plans])).to(dev)
    ws = sd.workspace(N, cfg.D)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    acc_h = torch.zeros((K, N), dtype=torch.int32, device=dev)
    nxt_h = torch.zeros((K, N), dtype=torch.int32, device=dev)
    lens_h = torch.zeros((K, N), dtype=torch.int32, device=dev)
    groups = []
    torch.cuda.synchronize()
    del keep
    ev = _events(K, 5)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for r in range(K):
        ev[r][0].record()
        order, uni, wid, nu = sd.group_by_len(pool.len, G)
        ev[r][1].record()
        sd.gather(pool, rect, order, G, uni, status=status)
        ev[r][2].record()
        sd.verify_greedy(logits[r], drafts[r], ws=ws, status=status, accept_len=acc_h[r], next_token=nxt_h[r])
        ev[r][3].record()
        sd.append(pool, kv_new[r], drafts[r], acc_h[r], nxt_h[r], status=status)
        ev[r][4].record()
        groups.append((order, uni, wid))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    if int(status.item()) != 0:
        raise RuntimeError("device status %d during the timed rounds" % int(status.item()))
    g_ms, ga_ms, v_ms, ap_ms = _ms(ev, 0, 1), _ms(ev, 1, 2), _ms(ev, 2, 3), _ms(ev, 3, 4)
    P = cfg.kv_pos_bytes
    lens = lens0.astype(np.int64).copy()
    gbytes, abytes, mixed = [], [], []
    accs = acc_h.cpu().numpy()
    for r in range(K):
        order, uni, wid = (t.cpu().numpy() for t in groups[r])
        gb = 0
        for g in range(ng):
            if uni[g]:
                continue
            rows = order[g * G:(g + 1) * G]
            gb += P * (int(lens[rows].sum()) + len(rows) * int(wid[g]))
        gbytes.append(gb)
        mixed.append(int((uni == 0).sum()))
        n = accs[r].astype(np.int64) + 1
        abytes.append(2 * P * int(n.sum()))
        lens = lens + n
    gbytes = np.array(gbytes, dtype=np.float64)
    vbytes = N * cfg.D1 * cfg.V * 2 + N * cfg.D * 4 + 8 * N
    ga_gbs = gbytes.sum() / (ga_ms.sum() * 1e-3) / 1e9 if gbytes.sum() > 0 else 0.0
    cpu = None
    if not args.no_cpu:
        del pool, rect, logits, kv_new
        torch.cuda.empty_cache()
        cpu = cpu_exspec(cfg, plans, lens0, min(args.cpu_rounds, K, 4))
    eq_bytes, eq_inplace = eqspec_pool_bytes(cfg, lens0, accs)
    ex_bytes = gbytes + np.array(abytes, dtype=np.float64)
    config = {"workload": "exspec: pool of %d sequences, batches of %d, D=%d, V=%d bf16 logits, KV %dx%dx%d bf16, 16 "
                          "distinct lengths in [512,4096], %d rounds" % (N, G, cfg.D, cfg.V, cfg.L, cfg.H, cfg.Dh, K),
              "pool": N, "group": G, "D": cfg.D, "V": cfg.V, "cap": cap, "global_batch": N}
    extra = {"verify": {"kernel": "k_verify_greedy", "achieved_gbs": vbytes / (v_ms.mean() * 1e-3) / 1e9,
                        "avg_launch_us": float(v_ms.mean() * 1e3)},
             "group_us": float(g_ms.mean() * 1e3), "append_us": float(ap_ms.mean() * 1e3),
             "append_gbs": float(np.sum(abytes) / (ap_ms.sum() * 1e-3) / 1e9),
             "gather_us": float(ga_ms.mean() * 1e3), "mixed_batches_per_round": mixed,
             "uniform_batches_per_round": [ng - m for m in mixed],
             "realign_share_of_round": float((ga_ms.sum() + g_ms.sum()) / total_ms),
             "vs_eqspec": {
                 "exspec_bytes_per_round": float(ex_bytes.mean()),
                 "exspec_bytes_round_1": float(ex_bytes[0]),
                 "eqspec_out_of_place_bytes_per_round": float(eq_bytes.mean()),
                 "eqspec_in_place_bytes_per_round": float(eq_inplace.mean()),
                 "exspec_over_eqspec": float(ex_bytes.sum() / eq_bytes.sum()),
                 "how": "EXSPEC: the gather of mixed batches plus the in-place append (algorithmic bytes of these "
                        "rounds); EQSPEC: the same pool held as fixed batches of %d consecutive rows, each a "
                        "left-padded rectangle realigned every round with the same accepted lengths "
                        "(out of place, and the in-place variant's moved bytes)" % G},
             "cycle": cycle_stats(accs, cfg.D, K / (total_ms * 1e-3)),
             "memory": device_memory(dev),
             "host": host_info()}
    return _line("EXSPEC pool rounds/sec and gather HBM GB/s (256-sequence pool)", K / (total_ms * 1e-3), K, W,
                 total_ms / K, "bf16", config,
                 _roof("k_gather", ga_gbs, float(gbytes.mean()), float(ga_ms.mean() * 1e3)), cpu, extra)


def bench_lifecycle(args, cfg):
    """Pool rounds with the sequence lifecycle: the exspec pool (256 slots, full
    at the start) and a queue of 256 more prompts (lengths uniform in the pool's
    range).  Each round: group the active sequences, gather the mixed batches,
    verify, append, finish sequences whose committed tokens hold the
    end-of-sequence id (planted at the stop position of 1 in 16 sequences per
    round) or that reach max_len, and admit queued prompts into the freed slots.
    The host reads the active count once per round to size the next one."""
    import numpy as np
    import torch
    import synth
    import synth.device as sdev
    import ragged_kv_realignment_amd as sd

    K = args.steps if args.steps is not None else cfg.rounds
    N, G, D1, EOS = cfg.B, cfg.group, cfg.D1, 2
    Q = N
    dev = torch.device("cuda", 0)
    tdt = sdev.TORCH_DT[cfg.kv_dtype]
    cap = max(cfg.cap, cfg.len_hi + K * D1)
    max_len = cap - D1
    lens0 = synth.lengths(cfg)
    pool = sd.SeqBuf.empty(cfg.L, N, cfg.H, cap, cfg.Dh, tdt, pool=True)
    sdev.fill_kv(cfg, pool.kv, torch.from_numpy(lens0).to(dev), 0, False)
    tok0, _, _ = synth.tokens_host(cfg, lens0, 0, False, cap=cap)
    pool.tokens.copy_(torch.from_numpy(tok0))
    pool.len.copy_(torch.from_numpy(lens0))
    rng = np.random.default_rng(cfg.seed)
    qlen = rng.integers(cfg.len_lo, cfg.len_hi + 1, Q).astype(np.int32)
    queue = sd.SeqBuf.empty(cfg.L, Q, cfg.H, cfg.len_hi, cfg.Dh, tdt, pool=True)
    sdev.fill_kv(cfg, queue.kv, torch.from_numpy(qlen).to(dev), 0, False)
    qtok, _, _ = synth.tokens_host(cfg, qlen, 0, False, rows=Q, cap=cfg.len_hi)
    queue.tokens.copy_(torch.from_numpy(qtok))
    queue.len.copy_(torch.from_numpy(qlen))
    sched = sd.Sched(N, active=range(N))
    ng = (N + G - 1) // G
    rect = sd.SeqBuf.empty(cfg.L, N, cfg.H, cap, cfg.Dh, tdt, groups=ng)
    logits = torch.empty((K, N, D1, cfg.V), dtype=sdev.TORCH_DT[cfg.logit_dtype], device=dev)
    drafts = []
    plants = []
    keep = []
    for r in range(K):
        plant, miss, draft = synth.plan_greedy(cfg, r)
        for b in np.nonzero(rng.random(N) < 1.0 / 16)[0]:
            row = b * D1 + int(miss[b])
            plant[row] = (EOS, -1, -1)
            if miss[b] < cfg.D and draft[b, miss[b]] == EOS:
                draft[b, miss[b]] = EOS + 1
        keep.append(sdev.fill_logits(cfg, r, plant, logits[r]))
        drafts.append(draft)
        plants.append(plant)
    host_drafts = drafts
    drafts = torch.from_numpy(np.stack(drafts)).to(dev)
    kv_new = torch.empty((K, cfg.L, 2, N, cfg.H, D1, cfg.Dh), dtype=tdt, device=dev)
    for r in range(K):
        sdev.fill_kvnew(cfg, r, kv_new[r])
    ws = sd.workspace(N, cfg.D)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    acc = torch.zeros(N, dtype=torch.int32, device=dev)
    nxt = torch.zeros(N, dtype=torch.int32, device=dev)
    retired = torch.zeros(N, dtype=torch.int32, device=dev)
    n_ret = torch.zeros(1, dtype=torch.int32, device=dev)
    admitted = torch.zeros(N, dtype=torch.int32, device=dev)
    n_adm = torch.zeros(1, dtype=torch.int32, device=dev)
    counts = torch.zeros((K, 3), dtype=torch.int32, device=dev)  # active, retired, admitted per round
    torch.cuda.synchronize()
    del keep
    ev = _events(K, 3)
    B = N
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for r in range(K):
        if B == 0:
            break
        ev[r][0].record()
        order, uni, wid, nu = sd.group_by_len(pool.len, G, ids=sched.active[:B])
        sd.gather(pool, rect, order, G, uni, status=status)
        sd.verify_greedy(logits[r, :B], drafts[r, :B], ws=ws, status=status, accept_len=acc[:B],
                         next_token=nxt[:B])
        kvn = kv_new[r] if B == N else kv_new[r, :, :, :B].contiguous()  # the active batch's entries
        sd.append(pool, kvn, drafts[r, :B], acc[:B], nxt[:B], rows=order, status=status)
        ev[r][1].record()
        sd.pool_finish(pool, sched, order, acc[:B], cfg.D, EOS, max_len, retired=retired, n_retired=n_ret,
                       status=status)
        sd.pool_admit(pool, sched, queue, admitted=admitted, n_admitted=n_adm, status=status)
        ev[r][2].record()
        counts[r, 0] = B
        counts[r, 1:2].copy_(n_ret)
        counts[r, 2:3].copy_(n_adm)
        B = int(sched.n_active.item())  # the host sizes the next round
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    if int(status.item()) != 0:
        raise RuntimeError("device status %d during the lifecycle rounds" % int(status.item()))
    cnt = counts.cpu().numpy()
    done = int((cnt[:, 0] > 0).sum())
    step_ms, life_ms = _ms(ev[:done], 0, 1), _ms(ev[:done], 1, 2)
    config = {"workload": "exspec pool with lifecycle: %d slots full at the start, %d queued prompts with lengths "
                          "U[%d,%d], batches of %d, D=%d, V=%d bf16, KV %dx%dx%d bf16, end-of-sequence planted at the "
                          "stop position of 1 in 16 sequences per round, max_len %d, %d rounds"
                          % (N, Q, cfg.len_lo, cfg.len_hi, G, cfg.D, cfg.V, cfg.L, cfg.H, cfg.Dh, max_len, K),
              "pool": N, "queue": Q, "group": G, "D": cfg.D, "V": cfg.V, "cap": cap, "global_batch": N}
    extra = {"finished_sequences": int(cnt[:, 1].sum()), "admitted_sequences": int(cnt[:, 2].sum()),
             "finished_per_s": float(cnt[:, 1].sum() / (total_ms * 1e-3)),
             "active_per_round": [int(x) for x in cnt[:done, 0]],
             "round_step_ms": float(step_ms.mean()), "lifecycle_us": float(life_ms.mean() * 1e3),
             "lifecycle_share_of_round": float(life_ms.sum() / total_ms)}
    cpu = None
    if not args.no_cpu:
        del pool, queue, rect, logits, kv_new
        torch.cuda.empty_cache()
        cpu = cpu_lifecycle(cfg, plants, host_drafts, lens0, tok0, qlen, qtok, cap, EOS, max_len,
                            min(args.cpu_rounds, done, 2))
    line = _line("EXSPEC pool rounds/sec with the sequence lifecycle (256-slot pool)", done / (total_ms * 1e-3),
                 done, 0, total_ms / max(done, 1), "bf16", config, None, cpu, extra)
    line["roofline"] = {"bound": "latency", "kernels": "k_pool_finish + k_pool_admit_plan + k_pool_admit_copy",
                        "avg_call_us": float(life_ms.mean() * 1e3), "note": "one-workgroup list updates plus "
                        "the admitted prompts' KV copy; the round's bytes are in the exspec line"}
    return line


def _oracle_pool_rounds(cfg, plans, lens0, rounds):
    """(grouping + verification seconds, layer-0 gather + append seconds) of
    the oracle over the first rounds of the pool chain."""
    import numpy as np
    import oracle
    import synth
    N, G = cfg.B, cfg.group
    kv = synth.kv_host(cfg, lens0, 0, False, layer0=0, nlayers=1)
    tok, _, _ = synth.tokens_host(cfg, lens0, 0, False)
    lens = lens0.copy()
    t_fix = t_lay = 0.0
    for r in range(rounds):
        plant, _, draft = plans[r]
        lg = synth.logits_host(cfg, r, plant)
        kvn = synth.kvnew_host(cfg, r, layer0=0, nlayers=1)
        t0 = time.perf_counter()
        order, uni, wid, nu = oracle.group_by_len(lens, G)
        acc, nxt, _ = oracle.verify_greedy(lg, draft, N, cfg.D, cfg.V)
        t1 = time.perf_counter()
        oracle.gather(kv, tok, lens, order, G, uni, cfg.cap)
        oracle.append(kv, tok, lens, np.arange(N), kvn, draft, acc, nxt)
        t2 = time.perf_counter()
        t_fix += t1 - t0
        t_lay += t2 - t1
    return t_fix, t_lay


def cpu_exspec(cfg, plans, lens0, rounds):
    """The oracle on the first rounds of the pool chain: grouping, verification of
    all sequences, gather and append of layer 0, scaled to all layers; the
    single-threaded build, and beside it the OpenMP build of the same source."""
    import oracle
    N = cfg.B
    t_fix, t_lay = _oracle_pool_rounds(cfg, plans, lens0, rounds)
    with oracle.threaded():
        threads = oracle.threads()
        m_fix, m_lay = _oracle_pool_rounds(cfg, plans, lens0, rounds)
    per, m_per = (t_fix + t_lay * cfg.L) / rounds, (m_fix + m_lay * cfg.L) / rounds
    return {"value": 1.0 / per, "unit": "rounds/s", "cores": 1, "kind": "oracle",
            "sample": "rounds 0-%d of the pool chain: grouping and greedy verify of all %d sequences (%.1f ms/round), "
                      "gather + append of layer 0 (%.1f ms/round) scaled by %d layers; single-threaded C oracle"
                      % (rounds - 1, N, 1e3 * t_fix / rounds, 1e3 * t_lay / rounds, cfg.L),
            "host_cpus": os.cpu_count(),
            "all_cores": {"value": 1.0 / m_per, "unit": "rounds/s", "cores": threads, "kind": "oracle (OpenMP build)",
                          "sample": "the same sample on %d threads: grouping and verify %.1f ms/round, layer 0 "
                                    "%.1f ms/round before scaling" % (threads, 1e3 * m_fix / rounds,
                                                                      1e3 * m_lay / rounds)}}


def cpu_lifecycle(cfg, plants, drafts, lens0, tok0, qlen, qtok, cap, eos, max_len, rounds):
    """The oracle on the first rounds of the lifecycle chain, with the same
    inputs: grouping of the active sequences, their greedy verification, the
    gather and append of layer 0, finishing and admission (the prompt copy of
    layer 0); the layer-0 work is scaled to all layers.  Single-threaded build,
    and the OpenMP build beside it."""
    import numpy as np
    import oracle
    import synth
    N, G, D = cfg.B, cfg.group, cfg.D
    Q, qcap = qtok.shape

    def run():
        kv = synth.kv_host(cfg, lens0, 0, False, layer0=0, nlayers=1, cap=cap)
        tok, lens = tok0.copy(), lens0.astype(np.int32).copy()
        qkv = synth.kv_host(cfg, qlen, 0, False, layer0=0, nlayers=1, rows=Q, cap=qcap)
        sched = oracle.Sched(N, range(N))
        t_fix = t_lay = 0.0
        for r in range(rounds):
            act = sched.active_list()
            B = len(act)
            lg = synth.logits_host(cfg, r, plants[r], nrows=B * cfg.D1)
            kvn = synth.kvnew_host(cfg, r, layer0=0, nlayers=1)[:, :, :B]
            t0 = time.perf_counter()
            order_l, uni, wid, nu = oracle.group_by_len(lens[act], G)
            order = act[order_l]
            acc, nxt, _ = oracle.verify_greedy(lg, drafts[r][:B], B, D, cfg.V)
            t1 = time.perf_counter()
            oracle.gather(kv, tok, lens, order, G, uni, cap)
            oracle.append(kv, tok, lens, order, kvn, drafts[r][:B], acc, nxt)
            t2 = time.perf_counter()
            oracle.pool_finish(tok, lens, sched, order, acc, D, eos, max_len)
            t3 = time.perf_counter()
            oracle.pool_admit(kv, tok, lens, sched, qkv, qtok, qlen)
            t4 = time.perf_counter()
            t_fix += (t1 - t0) + (t3 - t2)
            t_lay += (t2 - t1) + (t4 - t3)
        return t_fix, t_lay

    t_fix, t_lay = run()
    with oracle.threaded():
        threads = oracle.threads()
        m_fix, m_lay = run()
    per, m_per = (t_fix + t_lay * cfg.L) / rounds, (m_fix + m_lay * cfg.L) / rounds
    return {"value": 1.0 / per, "unit": "rounds/s", "cores": 1, "kind": "oracle",
            "sample": "rounds 0-%d of the lifecycle chain: grouping, greedy verify and finishing of the active "
                      "sequences (%.1f ms/round), gather + append + admission of layer 0 (%.1f ms/round) scaled by "
                      "%d layers; single-threaded C oracle" % (rounds - 1, 1e3 * t_fix / rounds,
                                                             1e3 * t_lay / rounds, cfg.L),
            "host_cpus": os.cpu_count(),
            "all_cores": {"value": 1.0 / m_per, "unit": "rounds/s", "cores": threads, "kind": "oracle (OpenMP build)",
                          "sample": "the same sample on %d threads" % threads}}


def eqspec_pool_bytes(cfg, lens0, accs):
    """Bytes per round of the same pool kept as EQSPEC rectangles instead: the
    256 sequences in fixed batches of `group` consecutive pool rows, each a
    left-padded rectangle realigned every round (unpad, append, repad out of
    place), P * (sum c + sum n + group * S') per batch; and the in-place
    variant's moved bytes, P * (2 * sum of moved rows' c + sum of shifts + 2 * sum n)."""
    import numpy as np
    N, G, P = cfg.B, cfg.group, cfg.kv_pos_bytes
    lens = lens0.astype(np.int64).copy()
    width = [int(lens[g:g + G].max()) for g in range(0, N, G)]
    out, inpl = [], []
    for acc in accs:
        n = acc.astype(np.int64) + 1
        tot = ip = 0
        for k, g in enumerate(range(0, N, G)):
            c, nb = lens[g:g + G], n[g:g + G]
            snew = int((c + nb).max())
            tot += P * (int(c.sum()) + int(nb.sum()) + len(c) * snew)
            shift = snew - width[k] - nb
            moved = (shift != 0) & (c > 0)
            ip += P * (2 * int(c[moved].sum()) + int(np.maximum(shift, 0).sum()) + 2 * int(nb.sum()))
            width[k] = snew
        out.append(tot)
        inpl.append(ip)
        lens = lens + n
    return np.array(out, dtype=np.float64), np.array(inpl, dtype=np.float64)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    torch.cuda.set_device(0)
    cfg = synth.CONFIGS[args.config]
    if cfg.name == "stoch":
        line = bench_stoch(args, cfg)
    elif cfg.name == "exspec" and args.lifecycle:
        line = bench_lifecycle(args, cfg)
    elif cfg.name == "exspec":
        line = bench_exspec(args, cfg)
    else:
        line = bench_chain(args, cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
