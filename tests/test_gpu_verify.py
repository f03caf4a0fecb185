"""GPU parity of verification: the HIP kernels against the oracle, bit-exact for
greedy, within the stated band for sampling."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.device as sdev
from tests.gpu_util import from_np_raw, say, to_np_raw

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_kv_realignment_amd as m
    return m


def _encode(rows_f32, enc):
    if enc == "f32":
        return rows_f32.astype(np.float32), torch.float32
    if enc == "f16":
        return rows_f32.astype(np.float16), torch.float16
    return (rows_f32.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16), torch.bfloat16


def _gpu_greedy(sd, host_rows, tdt, B, D, V, draft, row_stride=None, offset_elems=0):
    """Run the kernel on host rows [B*(D+1), V]; optional padded rows / misaligned base."""
    rs = V if row_stride is None else row_stride
    buf = np.zeros((B * (D + 1) * rs + offset_elems + 8,), dtype=host_rows.dtype)
    view = buf[offset_elems:offset_elems + B * (D + 1) * rs].reshape(B * (D + 1), rs)
    view[:, :V] = host_rows
    dev = from_np_raw(buf, tdt)
    logits = torch.as_strided(dev, (B, D + 1, V), (rs * (D + 1), rs, 1), offset_elems)
    tgt = torch.empty((B, D + 1), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt = sd.verify_greedy(logits, torch.from_numpy(np.ascontiguousarray(draft, np.int32)).cuda(),
                                status=status, target_tok=tgt)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy(), tgt.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("enc", ["f32", "f16", "bf16"])
def test_greedy_ties_signed_zero_and_infinities(sd, enc):
    say("greedy ties", enc)
    V, D = 3000, 3
    rows = np.full((D + 1, V), -3.0, np.float32)
    rows[0, [2047, 5, 2999, 1000]] = 1.5
    rows[1, :] = -1.0
    rows[1, 2500] = -0.0
    rows[1, 2600] = 0.0
    rows[2, :] = -np.inf
    rows[3, :] = 0.25
    rows[3, 2999] = np.inf
    host, tdt = _encode(rows, enc)
    draft = np.array([[5, 2500, 0]], np.int32)
    acc, nxt, tgt, st = _gpu_greedy(sd, host, tdt, 1, D, V, draft)
    oacc, onxt, otgt = oracle.verify_greedy(host, draft, 1, D, V)
    assert list(otgt[0]) == [5, 2500, 0, 2999]
    assert np.array_equal(tgt, otgt) and np.array_equal(acc, oacc) and np.array_equal(nxt, onxt)
    assert st == 0


@pytest.mark.parametrize("enc", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 0, 1), (1, 0, 7), (3, 2, 9), (5, 4, 1000), (2, 6, 4099), (7, 3, 70001),
                                   (1, 0, 196608), (120, 4, 3001), (100, 5, 20480), (40000, 3, 7)])
def test_greedy_discrete_random(sd, enc, shape):
    """Logits drawn from a few values (many exact ties, -0 and +0), odd V, a
    ragged last vector, several workgroups per row, many rows."""
    B, D, V = shape
    say("greedy discrete", enc, shape)
    rng = np.random.default_rng(B * 1000 + D * 10 + V)
    vals = np.array([-7.0, -0.0, 0.0, 0.5, 2.0, 2.0], np.float32)
    rows = vals[rng.integers(0, len(vals), (B * (D + 1), V))]
    host, tdt = _encode(rows, enc)
    t0 = np.argmax(rows.reshape(B, D + 1, V), axis=-1)
    draft = np.where(rng.random((B, D)) < 0.8, t0[:, :D], rng.integers(0, V, (B, D))).astype(np.int32)
    acc, nxt, tgt, st = _gpu_greedy(sd, host, tdt, B, D, V, draft)
    oacc, onxt, otgt = oracle.verify_greedy(host, draft, B, D, V)
    assert np.array_equal(tgt, otgt)
    assert np.array_equal(acc, oacc) and np.array_equal(nxt, onxt)


@pytest.mark.parametrize("enc", ["f32", "bf16"])
def test_greedy_strided_and_misaligned_rows(sd, enc):
    """Rows with padding between them and a base that is not 16-byte aligned
    (the kernel's scalar path)."""
    B, D, V = 4, 3, 5003
    rng = np.random.default_rng(9)
    rows = rng.standard_normal((B * (D + 1), V)).astype(np.float32)
    host, tdt = _encode(rows, enc)
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    oacc, onxt, otgt = oracle.verify_greedy(host, draft, B, D, V)
    for rs, off in ((5008, 0), (5011, 1), (V, 3)):
        say("greedy strided", enc, rs, off)
        acc, nxt, tgt, _ = _gpu_greedy(sd, host, tdt, B, D, V, draft, row_stride=rs, offset_elems=off)
        assert np.array_equal(tgt, otgt) and np.array_equal(acc, oacc) and np.array_equal(nxt, onxt)


def test_greedy_draft_out_of_range_sets_status(sd):
    say("greedy draft range")
    B, D, V = 2, 3, 100
    rows = np.random.default_rng(1).standard_normal((B * (D + 1), V)).astype(np.float32)
    draft = np.array([[-1, 3, 4], [1, 2, 100]], np.int32)
    acc, nxt, tgt, st = _gpu_greedy(sd, rows, torch.float32, B, D, V, draft)
    oacc, onxt, _ = oracle.verify_greedy(rows, draft, B, D, V)
    assert np.array_equal(acc, oacc) and np.array_equal(nxt, onxt)
    assert st & sd.S_DRAFT_RANGE


def test_greedy_workspace_reuse_many_calls(sd):
    """One workspace serves consecutive calls (it is left cleared)."""
    say("greedy workspace reuse")
    B, D, V = 6, 4, 20000
    ws = sd.workspace(B, D)
    rng = np.random.default_rng(3)
    for k in range(5):
        rows = rng.standard_normal((B * (D + 1), V)).astype(np.float32)
        draft = rng.integers(0, V, (B, D)).astype(np.int32)
        dev = torch.from_numpy(rows).cuda().view(B, D + 1, V)
        acc, nxt = sd.verify_greedy(dev, torch.from_numpy(draft).cuda(), ws=ws)
        oacc, onxt, _ = oracle.verify_greedy(rows, draft, B, D, V)
        assert np.array_equal(acc.cpu().numpy(), oacc) and np.array_equal(nxt.cpu().numpy(), onxt)
    assert int(ws.count_nonzero().item()) == 0


@pytest.mark.parametrize("name", ["tiny", "7b-mha", "8b-gqa", "exspec"])
def test_greedy_workload_rounds(sd, name):
    """Generated workloads at full size: every row of several rounds, bit-exact,
    and the planted closed form (accepted length = designed first mismatch)."""
    cfg = synth.CONFIGS[name]
    rounds = 3 if name != "exspec" else 1
    for r in range(rounds):
        say("greedy workload", name, "round", r)
        plant, miss, draft = synth.plan_greedy(cfg, r)
        logits = torch.empty((cfg.B, cfg.D1, cfg.V), dtype=sdev.TORCH_DT[cfg.logit_dtype], device="cuda")
        keep = sdev.fill_logits(cfg, r, plant, logits)
        tgt = torch.empty((cfg.B, cfg.D1), dtype=torch.int32, device="cuda")
        acc, nxt = sd.verify_greedy(logits, torch.from_numpy(draft).cuda(), target_tok=tgt)
        torch.cuda.synchronize()
        del keep
        host = synth.logits_host(cfg, r, plant)
        assert np.array_equal(to_np_raw(logits).reshape(host.shape).view(np.uint8), host.view(np.uint8)), \
            "device generator differs from host generator"
        oacc, onxt, otgt = oracle.verify_greedy(host, draft, cfg.B, cfg.D, cfg.V)
        assert np.array_equal(tgt.cpu().numpy(), otgt)
        assert np.array_equal(acc.cpu().numpy(), oacc) and np.array_equal(nxt.cpu().numpy(), onxt)
        assert np.array_equal(oacc, miss)


# ------------------------------------------------------------------ sampled

BAND = 1e-6


def _admissible_draw(p_row, q_row, u, j, band=BAND):
    """Is id j an admissible inverse-CDF draw for uniform u (oracle arithmetic,
    fp64 cumulative mass, decisions within band*T of a boundary accepted)?"""
    w = np.maximum(p_row.astype(np.float64) - (q_row.astype(np.float64) if q_row is not None else 0.0), 0.0)
    if not w.sum() > 0:
        w = np.maximum(p_row.astype(np.float64), 0.0)
    c = np.cumsum(w)
    T = c[-1]
    t = float(u) * T
    lo = c[j - 1] if j > 0 else 0.0
    return w[j] > 0 and lo - band * T <= t < c[j] + band * T


def _check_sampled(p, q, draft, u_acc, u_draw, acc, nxt):
    oacc, onxt, _ = oracle.verify_sample(p, q, draft, u_acc, u_draw)
    assert np.array_equal(acc, oacc), "acceptance is exact on both sides"
    D = q.shape[1]
    n_amb = 0
    for b in np.nonzero(nxt != onxt)[0]:
        a = acc[b]
        qrow = q[b, a] if a < D else None
        assert _admissible_draw(p[b, a], qrow, u_draw[b, a], nxt[b]), "row %d: draw outside the band" % b
        n_amb += 1
    return n_amb


def test_sample_stochastic_workload(sd):
    cfg = synth.CONFIGS["stoch"]
    say("sample workload stoch")
    p, q, draft, u_acc, u_draw = synth.sampled_round(cfg, 0)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in (p, q, draft, u_acc, u_draw)), status=status)
    torch.cuda.synchronize()
    n_amb = _check_sampled(p, q, draft, u_acc, u_draw, acc.cpu().numpy(), nxt.cpu().numpy())
    assert n_amb == 0
    assert int(status.item()) == 0


@pytest.mark.parametrize("seed", range(6))
def test_sample_random_small(sd, seed):
    rng = np.random.default_rng(100 + seed)
    B, D, V = int(rng.integers(1, 40)), int(rng.integers(0, 9)), int(rng.integers(1, 3000))
    say("sample random", seed, B, D, V)
    p = rng.random((B, D + 1, V)).astype(np.float32)
    p[rng.random(p.shape) < 0.3] = 0.0
    p[..., 0] += 1e-3
    p /= p.sum(-1, keepdims=True)
    q = rng.random((B, D, V)).astype(np.float32)
    q[rng.random(q.shape) < 0.3] = 0.0
    q[..., -1] += 1e-3
    q /= q.sum(-1, keepdims=True)
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    if seed == 0 and D > 0:
        q[0, 0] = p[0, 0]  # p == q at a position: certain acceptance
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in (p, q, draft, u_acc, u_draw)))
    torch.cuda.synchronize()
    _check_sampled(p, q, draft, u_acc, u_draw, acc.cpu().numpy(), nxt.cpu().numpy())


@pytest.mark.parametrize("V", [32000, 151936, 100003, 65537, 4097])
def test_sample_many_splits(sd, V):
    """Rows spread over many workgroups (up to 16 splits of 256 runs; an odd V
    takes the scalar path): peaked and flat rows, draws near the top and the
    bottom of the cumulative mass, all against the oracle within the band."""
    rng = np.random.default_rng(V)
    B, D = 6, 3
    say("sample many splits", V)
    logits = rng.standard_normal((B, D + 1, V)) * np.array([0.5, 2.0, 4.0, 1.0, 3.0, 0.1])[:, None, None]
    p = np.exp(logits - logits.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    ql = logits[:, :D] + 0.5 * rng.standard_normal((B, D, V))
    q = np.exp(ql - ql.max(-1, keepdims=True))
    q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    qd = q.astype(np.float64)
    qd /= qd.sum(-1, keepdims=True)
    draft = np.array([[int(rng.choice(V, p=qd[b, i])) for i in range(D)] for b in range(B)], np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    u_draw[0] = 1.0 - 2.0 ** -24   # the top of the mass
    u_draw[1] = 0.0                # the bottom
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in (p, q, draft, u_acc, u_draw)), status=status)
    torch.cuda.synchronize()
    _check_sampled(p, q, draft, u_acc, u_draw, acc.cpu().numpy(), nxt.cpu().numpy())
    assert int(status.item()) == 0


@pytest.mark.parametrize("V", [1 << 26, (1 << 24) + 3])
def test_sample_long_runs(sd, V):
    """Vocabularies far past the 16 x 256 runs a row is cut into, so every run
    holds thousands of ids (16,384 at V = 2^26; an odd V takes the scalar
    path): sums and the draw's walk over long runs, draws at the top, the
    bottom and the middle of the mass, against the oracle within the band."""
    rng = np.random.default_rng(V % 1000)
    B, D = 3, 1
    say("sample long runs", V)
    p = rng.random((B, D + 1, V), dtype=np.float32)
    p[:, :, : V // 3] *= 0.01  # a third of the ids carry little mass
    p /= p.sum(-1, keepdims=True, dtype=np.float64).astype(np.float32)
    q = rng.random((B, D, V), dtype=np.float32)
    q /= q.sum(-1, keepdims=True, dtype=np.float64).astype(np.float32)
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    u_acc = np.full((B, D), 0.999, np.float32)  # rejections mostly: the residual draw
    u_draw = np.array([[1.0 - 2.0 ** -24] * (D + 1), [0.0] * (D + 1), [0.5] * (D + 1)], np.float32)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in (p, q, draft, u_acc, u_draw)), status=status)
    torch.cuda.synchronize()
    _check_sampled(p, q, draft, u_acc, u_draw, acc.cpu().numpy(), nxt.cpu().numpy())
    assert int(status.item()) == 0


def test_sample_workspace_reused_across_shapes(sd):
    """One workspace, sized for the most rows, serves calls of different
    vocabularies and batch sizes one after another: each row's counter and runs
    sit at a place that depends on the row alone, every call leaves its
    counters cleared and writes every run sum it reads."""
    rng = np.random.default_rng(5150)
    shapes = ((40, 4, 151936), (3, 2, 1000), (40, 4, 32000), (1, 0, 7), (17, 4, 151936))
    need = max(int(sd.lib().specdec_verify_sample_workspace_bytes(*sh)) for sh in shapes)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert sd.lib().specdec_workspace_init(ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream) == 0
    for B, D, V in shapes:
        say("sample workspace reuse", B, D, V)
        p = rng.random((B, D + 1, V)).astype(np.float32)
        p /= p.sum(-1, keepdims=True)
        q = rng.random((B, D, V)).astype(np.float32)
        q /= q.sum(-1, keepdims=True)
        draft = rng.integers(0, V, (B, D)).astype(np.int32)
        u_acc = rng.random((B, D)).astype(np.float32)
        u_draw = rng.random((B, D + 1)).astype(np.float32)
        acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in (p, q, draft, u_acc, u_draw)), ws=ws)
        torch.cuda.synchronize()
        _check_sampled(p, q, draft, u_acc, u_draw, acc.cpu().numpy(), nxt.cpu().numpy())


def test_sample_longest_draft(sd):
    """D = 255, the longest draft: a row that accepts every draft (p = q) draws
    its bonus with u_draw[255]; a row rejected at position 200 draws there."""
    rng = np.random.default_rng(2550)
    B, D, V = 3, 255, 300
    say("sample D=255")
    p = rng.random((B, D + 1, V)).astype(np.float32)
    p /= p.sum(-1, keepdims=True)
    q = p[:, :D].copy()
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    u_acc = rng.random((B, D)).astype(np.float32)
    q[1, 200] = 0.0
    q[1, 200, draft[1, 200]] = 1.0          # q puts all mass on the draft
    p[1, 200, draft[1, 200]] = 0.0          # which p never takes: certain rejection
    p[1, 200] /= p[1, 200].sum()
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in (p, q, draft, u_acc, u_draw)))
    torch.cuda.synchronize()
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    assert acc[0] == D and acc[2] == D and acc[1] == 200
    _check_sampled(p, q, draft, u_acc, u_draw, acc, nxt)
    with pytest.raises(sd.SpecDecError):  # D = 256 is past the limit
        sd.verify_sample(*(torch.zeros(sh, device="cuda") for sh in ((1, 257, 8), (1, 256, 8))),
                         torch.zeros((1, 256), dtype=torch.int32, device="cuda"),
                         torch.zeros((1, 256), device="cuda"), torch.zeros((1, 257), device="cuda"))


def test_sample_worked_split(sd):
    """The newsletter page's 40/60 example through the kernel, with stratified uniforms."""
    say("sample worked split")
    p = np.array([0.4, 0.6], np.float32)
    q = np.array([0.8, 0.2], np.float32)
    drafts = np.array([0] * 80 + [1] * 20, np.int32)[:, None]
    u_acc = np.concatenate([(np.arange(80) + 0.5) / 80, (np.arange(20) + 0.5) / 20]).astype(np.float32)[:, None]
    u_draw = ((np.arange(200) + 0.5) / 200).astype(np.float32).reshape(100, 2)
    P = np.broadcast_to(p, (100, 2, 2)).copy()
    Q = np.broadcast_to(q, (100, 1, 2)).copy()
    acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in (P, Q, drafts, u_acc, u_draw)))
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    first = np.where(acc == 1, drafts[:, 0], nxt)
    assert int(np.sum(first == 0)) == 40 and int(np.sum(first == 1)) == 60


def test_sample_zero_row_status(sd):
    """A position whose target probabilities are all zero: the draft is rejected
    (0.5 * q(x) > p(x) = 0), the residual and its fallback are empty, so the
    draw yields id 0 and the PROB status bit; the oracle agrees."""
    say("sample zero row")
    B, D, V = 1, 1, 16
    p = np.zeros((B, D + 1, V), np.float32)
    q = np.zeros((B, D, V), np.float32)
    q[0, 0, 3] = 1.0
    args = (p, q, np.array([[3]], np.int32), np.full((1, 1), 0.5, np.float32), np.zeros((1, 2), np.float32))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in args), status=status)
    oacc, onxt, _ = oracle.verify_sample(*args)
    assert acc.item() == oacc[0] == 0 and nxt.item() == onxt[0] == 0
    assert int(status.item()) & sd.S_PROB


@pytest.mark.parametrize("V", [32000, 151936, 4097])
def test_sample_zero_residual_falls_back_to_p(sd, V):
    """Unnormalised inputs where p = q / 2 at the first position: u = 0.9
    rejects the draft there, max(0, p - q) has no mass, and the draw falls back
    to p at that position (runs of 8 ids walked from registers, longer runs,
    and the scalar path)."""
    rng = np.random.default_rng(77 + V)
    B, D = 5, 2
    say("sample zero residual", V)
    q = rng.random((B, D, V)).astype(np.float32)
    q /= q.sum(-1, keepdims=True)
    p = rng.random((B, D + 1, V)).astype(np.float32)
    p /= p.sum(-1, keepdims=True)
    p[:, 0] = 0.5 * q[:, 0]
    draft = rng.integers(0, V, (B, D)).astype(np.int32)
    u_acc = np.full((B, D), 0.9, np.float32)
    u_draw = rng.random((B, D + 1)).astype(np.float32)
    u_draw[0, 0] = 1.0 - 2.0 ** -24
    u_draw[1, 0] = 0.0
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt = sd.verify_sample(*(torch.from_numpy(x).cuda() for x in (p, q, draft, u_acc, u_draw)), status=status)
    torch.cuda.synchronize()
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    assert np.all(acc == 0)
    _check_sampled(p, q, draft, u_acc, u_draw, acc, nxt)
    assert int(status.item()) == 0


def test_greedy_longest_draft(sd):
    """D = 255, the longest draft the kernel accepts (D + 1 = 256 positions)."""
    say("greedy D=255")
    B, D, V = 2, 255, 300
    rng = np.random.default_rng(255)
    rows = rng.standard_normal((B * (D + 1), V)).astype(np.float32)
    t = np.argmax(rows.reshape(B, D + 1, V), axis=-1)
    draft = t[:, :D].copy().astype(np.int32)
    draft[1, 200] = (draft[1, 200] + 1) % V
    acc, nxt, tgt, _ = _gpu_greedy(sd, rows, torch.float32, B, D, V, draft)
    oacc, onxt, otgt = oracle.verify_greedy(rows, draft, B, D, V)
    assert list(oacc) == [255, 200]
    assert np.array_equal(tgt, otgt) and np.array_equal(acc, oacc) and np.array_equal(nxt, onxt)
    with pytest.raises(sd.SpecDecError):  # D = 256 is past the limit
        _gpu_greedy(sd, np.zeros((2 * 257, V), np.float32), torch.float32, 2, 256, V, np.zeros((2, 256), np.int32))


def test_caller_outputs_are_checked_before_launch(sd):
    """Outputs the caller supplies must be int32 (float32 for the cutoff),
    contiguous, on the logits' device and large enough, and a SeqBuf's lengths
    and width must fit its rows: otherwise the binding raises before anything
    is launched, so no kernel reads or writes past them."""
    say("caller outputs checked")
    B, D, V = 4, 3, 64
    logits = torch.zeros((B, D + 1, V), dtype=torch.float32, device="cuda")
    draft = torch.zeros((B, D), dtype=torch.int32, device="cuda")
    i32 = lambda n: torch.zeros(n, dtype=torch.int32, device="cuda")
    bad = [dict(accept_len=i32(B - 1)), dict(next_token=i32(B - 1)), dict(target_tok=i32(B * (D + 1) - 1)),
           dict(status=torch.zeros(1, dtype=torch.float32, device="cuda")), dict(status=i32(0)),
           dict(accept_len=torch.zeros(B, dtype=torch.int64, device="cuda")),
           dict(next_token=i32(2 * B)[::2]), dict(accept_len=torch.zeros(B, dtype=torch.int32))]
    for kw in bad:
        with pytest.raises(ValueError):
            sd.verify_greedy(logits, draft, **kw)
    acc, nxt = sd.verify_greedy(logits, draft, accept_len=i32(B), next_token=i32(B + 3), status=i32(1))
    torch.cuda.synchronize()
    assert acc.shape == (B,) and np.array_equal(acc.cpu().numpy(), np.full(B, D))  # all-equal rows: id 0 wins
    with pytest.raises(ValueError):
        sd.group_by_len(i32(16), 4, order=i32(15))
    with pytest.raises(ValueError):
        sd.verify_sample(torch.zeros((B, D + 1, V), device="cuda"), torch.zeros((B, D, V), device="cuda"), draft,
                         torch.zeros((B, D), device="cuda"), torch.zeros((B, D + 1), device="cuda"),
                         accept_len=i32(1))
    kv = torch.zeros((1, 2, 3, 1, 8, 8), dtype=torch.float16, device="cuda")
    tok = torch.zeros((3, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):  # one length per row
        sd.SeqBuf(kv, tok, i32(2))
    with pytest.raises(ValueError):  # an empty width
        sd.SeqBuf(kv, tok, i32(3), width=i32(0))
    with pytest.raises(ValueError):  # lengths on the host
        sd.SeqBuf(kv, tok, torch.zeros(3, dtype=torch.int32))


def test_greedy_full_shape_unplanted_natural_ties(sd):
    """Full-shape 8b-gqa rounds (B=16, D=5, V=151936 bf16) with unplanted N(0,2)
    logits: the maximum lies wherever the draws put it, and bf16's coarse grid
    makes it tie in several rows, at ids more than one split of the vocabulary
    apart (8192 ids is the largest split the launcher uses).  The oracle decides
    every target choice; the drafts follow its choices up to each row's
    designed first mismatch."""
    cfg = synth.CONFIGS["8b-gqa"]
    B, D, V = cfg.B, cfg.D, cfg.V
    cross_rows = 0
    for rnd in range(200, 204):   # rounds past the chain's: fresh draws
        say("greedy unplanted full shape", rnd)
        host = synth.logits_host(cfg, rnd, None, nrows=B * cfg.D1)
        f = (host.astype(np.uint32) << 16).view(np.float32)
        top = f.max(axis=1, keepdims=True)
        for row in np.nonzero((f == top).sum(axis=1) > 1)[0]:
            ids = np.nonzero(f[row] == top[row])[0]
            cross_rows += int(ids.max() - ids.min() >= 8192)
        _, _, tgt = oracle.verify_greedy(host, np.zeros((B, D), np.int32), B, D, V)
        _, miss, _ = synth.plan_greedy(cfg, rnd)
        draft = np.array(tgt[:, :D], np.int32)
        for b in range(B):
            if miss[b] < D:
                draft[b, miss[b]] = (tgt[b, miss[b]] + 1) % V
        acc, nxt, gtgt, st = _gpu_greedy(sd, host, torch.bfloat16, B, D, V, draft)
        oacc, onxt, otgt = oracle.verify_greedy(host, draft, B, D, V)
        assert np.array_equal(oacc, np.minimum(miss, D))
        assert np.array_equal(gtgt, otgt) and np.array_equal(acc, oacc) and np.array_equal(nxt, onxt)
        assert st == 0
    assert cross_rows >= 10, "the draws should tie at the maximum across splits in several rows"


def test_greedy_max_vocab(sd):
    """The largest vocabulary the call takes, 2^30 ids (one batch row, D = 1:
    two bf16 rows of 2 GiB, 131,072 workgroups per row): random finite logits
    below 2 in magnitude, the maximum 3.0 planted at three ids of row 0 (the
    lowest, 5, far from the others, so splits across the whole row compete) and
    at the last id of row 1 (the bonus)."""
    B, D, V = 1, 1, 1 << 30
    say("greedy max vocab", V)
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 16, size=(B * (D + 1), V), dtype=np.uint16)
    bits &= np.uint16(0xBFFF)  # exponent at most 127: finite, |x| < 2
    bits[0, [V - 1, V // 2 + 7, 5]] = np.uint16(0x4040)  # 3.0
    bits[1, V - 1] = np.uint16(0x4040)
    draft = np.array([[5]], np.int32)
    logits = torch.from_numpy(bits).cuda().view(torch.bfloat16).reshape(B, D + 1, V)
    tgt = torch.empty((B, D + 1), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc, nxt = sd.verify_greedy(logits, torch.from_numpy(draft).cuda(), status=status, target_tok=tgt)
    torch.cuda.synchronize()
    oacc, onxt, otgt = oracle.verify_greedy(bits, draft, B, D, V)
    assert np.array_equal(otgt, [[5, V - 1]])
    assert np.array_equal(tgt.cpu().numpy(), otgt) and int(status.item()) == 0
    assert np.array_equal(acc.cpu().numpy(), oacc) and np.array_equal(nxt.cpu().numpy(), onxt)
    assert int(oacc[0]) == 1 and int(onxt[0]) == V - 1
