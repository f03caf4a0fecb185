"""The seeded generator: encodings agree with library conversions and the
value distributions are what the workloads state."""
import numpy as np
import pytest
import torch

import synth


@pytest.mark.parametrize("sigma", [1.0, 2.0, 1e-4, 3e-6])
def test_f16_encoding_is_round_to_nearest_even(sigma):
    n = 400_000
    f32 = synth.normals(synth.F32, 9, 2, 0, n, sigma)
    f16 = synth.normals(synth.F16, 9, 2, 0, n, sigma)
    assert np.array_equal(f16.view(np.uint16), f32.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("sigma", [1.0, 2.0, 1e-30])
def test_bf16_encoding_is_round_to_nearest_even(sigma):
    n = 400_000
    f32 = synth.normals(synth.F32, 9, 2, 0, n, sigma)
    bf = synth.normals(synth.BF16, 9, 2, 0, n, sigma)
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, ref)


def test_normal_and_uniform_shapes():
    z = synth.normals(synth.F32, 4, 4, 0, 1_000_000).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    assert np.abs(z).max() < 6.0
    u = synth.uniforms(4, 7, 0, 1_000_000)
    assert u.min() >= 0.0 and u.max() < 1.0 and abs(u.mean() - 0.5) < 0.01
    assert np.array_equal(u, synth.uniforms(4, 7, 0, 1_000_000))
    assert not np.array_equal(u, synth.uniforms(4, 7, 1, 1_000_000))


def test_workload_lengths_and_caps():
    for name, cfg in synth.CONFIGS.items():
        lens = synth.lengths(cfg)
        assert lens.shape == (cfg.B,)
        assert lens.min() >= cfg.len_lo and lens.max() <= cfg.len_hi
        assert cfg.cap >= cfg.len_hi + cfg.rounds * cfg.D1
    lens = synth.lengths(synth.CONFIGS["exspec"])
    vals, counts = np.unique(lens, return_counts=True)
    assert len(vals) == 16 and np.all(counts == 16)


def test_plan_shapes_and_geometric_rate():
    cfg = synth.CONFIGS["7b-mha"]
    ks = np.concatenate([synth.plan_greedy(cfg, r)[1] for r in range(400)])
    # P(k = 0) = p for the geometric first mismatch
    assert abs(np.mean(ks == 0) - cfg.plan_p) < 0.05
    assert ks.min() >= 0 and ks.max() <= cfg.D
    plant, miss, draft = synth.plan_greedy(cfg, 0)
    assert plant.shape == (cfg.B * cfg.D1, 3) and draft.shape == (cfg.B, cfg.D)
    extra = plant[:, 1:]
    assert np.all((extra == -1) | (extra > plant[:, :1]))


def test_logit_rows_hold_planted_maximum():
    cfg = synth.CONFIGS["8b-gqa"]
    plant, _, _ = synth.plan_greedy(cfg, 0)
    lg = synth.logits_host(cfg, 0, plant, nrows=4)
    f = (lg.astype(np.uint32) << 16).view(np.float32)
    for r in range(4):
        assert f[r, plant[r, 0]] == cfg.plant_value
        others = np.delete(f[r], [i for i in plant[r] if i >= 0])
        assert others.max() < cfg.plant_value
        assert abs(others.std() - cfg.sigma) < 0.05
