"""The seeded input generator: determinism, distributions, bf16 rounding."""
import numpy as np
import pytest
import torch

from synth import (TINY_F32, CLIP_5S, SEQ_60S, STREAM_60S, STRESS_B4, WORKLOADS,
                   head_inputs, f32_to_bf16_bits, bf16_bits_to_f32, full_inputs)


def test_same_seed_same_bits():
    a = head_inputs(TINY_F32, 0, 1)
    b = head_inputs(TINY_F32, 0, 1)
    for key in ("q", "k", "v", "gamma", "beta"):
        assert np.array_equal(a[key], b[key])
    c = head_inputs(TINY_F32, 0, 0)
    assert not np.array_equal(a["q"], c["q"])


def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(3))
    x = rng.standard_normal(1 << 16).astype(np.float32) * np.float32(3e-3)
    # exact ties and a few specials that stay finite
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 2.0 ** -130], np.float32)
    x = np.concatenate([x, ties])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_table():
    assert STREAM_60S.stream_chunks == tuple([40] * 24 + [1])
    assert sum(STREAM_60S.stream_chunks) == SEQ_60S.T == 961
    assert SEQ_60S.state_std == 0.02 and CLIP_5S.state_std is None
    assert abs(SEQ_60S.key_scale - 1 / np.sqrt(128 * 880)) < 1e-15
    assert set(WORKLOADS) == {"tiny_f32", "clip5s_bf16", "seq60s_720p_bf16", "stream60s_bf16",
                              "stress_b4_bf16"}


def test_distributions_small_sample():
    w = CLIP_5S.with_(T=4)
    d = head_inputs(w, 0, 3)
    k = bf16_bits_to_f32(d["k"]).astype(np.float64)
    # keys scaled by 1/sqrt(D*S): E[||K_t||_F^2] = 1
    fro = (k ** 2).sum(axis=(1, 2))
    assert np.all(np.abs(fro - 1.0) < 0.02)
    assert np.all((d["gamma"] >= 0.95) & (d["gamma"] <= 1.0))
    assert np.all((d["beta"] > 0) & (d["beta"] < 1))
    q = bf16_bits_to_f32(d["q"])
    assert abs(q.std() - 1.0) < 0.01


def test_stress_boost_rows():
    w = STRESS_B4.with_(T=3)
    d = head_inputs(w, 1, 2)
    k = bf16_bits_to_f32(d["k"]).astype(np.float64) * np.sqrt(w.D * w.S)
    for t in range(w.T):
        rms = np.sqrt((k[t] ** 2).mean(axis=1))
        assert (rms > 2.5).sum() == 88
    assert np.all((d["beta"] >= 0.9) & (d["beta"] <= 1.0))
    assert np.all(d["gamma"] >= 0.999)


def test_full_inputs_stack_heads():
    full = full_inputs(TINY_F32, workers=1)
    h1 = head_inputs(TINY_F32, 0, 1)
    assert full["q"].shape == (1, 2, 8, 16, 32)
    assert np.array_equal(full["k"][0, 1], h1["k"])
    assert full["state"] is None
