"""The seeded input generator: determinism, bf16 rounding, per-expert seeds,
and the realised expert-load skew of the medium workload (through the oracle)."""
import numpy as np
import pytest

import moe_synth
import oracle
from _layers import custom


def test_deterministic_bytes():
    w = moe_synth.get("tiny")
    a, b = moe_synth.generate(w), moe_synth.generate(w)
    for k, v in a.items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(v, b[k]), k
    assert a["x"].shape == (128, 64) and a["x"].dtype == np.float32
    assert a["w_gate"].shape == (8, 128, 64) and a["w_down"].shape == (8, 64, 128)
    assert a["bias"] is None
    assert np.all(np.abs(a["w_gate"]) <= 1 / 8) and np.all(np.abs(a["w_down"]) <= 1 / np.sqrt(128))


def test_bf16_round_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -2.5, 3.0e38, 1e-40], np.float32)
    bits = moe_synth.f32_to_bf16_bits(f)
    back = moe_synth.bf16_bits_to_f32(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0                      # tie -> even
    assert back[2] == 1.0 + 4 * 2 ** -8         # tie -> even (up)
    assert back[3] == 1.0 + 2 ** -7             # above the tie -> up
    assert back[4] == -2.5
    # nearest: no other bf16 value is closer than the chosen one
    for v, r in zip(f.astype(np.float64), back.astype(np.float64)):
        ulp = 2.0 ** (np.floor(np.log2(abs(v))) - 7) if v != 0 and abs(v) > 1e-38 else 2.0 ** -133
        assert abs(v - r) <= ulp / 2 + 1e-300


def test_expert_regenerates_alone():
    w = moe_synth.get("small")
    a = moe_synth.generate(w)
    e = 3
    g = np.random.Generator(np.random.PCG64(moe_synth.expert_seed(w, e, 2)))
    v = g.standard_normal(w.d * w.d_ff, dtype=np.float32) * np.float32(w.w_std)
    assert np.array_equal(moe_synth.f32_to_bf16_bits(v).reshape(w.d, w.d_ff), a["w_down"][e])


def test_workload_table():
    W = moe_synth.WORKLOADS
    assert (W["small"].E, W["small"].K, W["small"].d_ff) == (4, 2, 1376)
    assert W["medium"].d_shared == 2 * 1408 and W["large_prefill"].rows == 16384 * 8
    assert W["large_decode"].T == 64 and W["latent"].d_e == 1024
    assert W["tiny"].route == "softmax_topk" and W["latent"].route == "sigmoid_bias"


def test_medium_router_skew():
    """Realised loads of the skewed workload: 4 empty experts, the busiest
    expert far above the mean, log-log slope of load vs rank about -1.1."""
    w = moe_synth.get("medium")
    a = moe_synth.generate(w, experts=False)
    idx, g, gap, _ = oracle.Oracle(w, a).route()
    counts = np.bincount(idx.ravel(), minlength=w.E)
    assert counts.sum() == w.T * w.K
    assert (counts == 0).sum() == moe_synth.ZIPF_EMPTY
    loads = np.sort(counts)[::-1]
    nz = loads[loads > 0]
    slope = np.polyfit(np.log(np.arange(1, len(nz) + 1)), np.log(nz), 1)[0]
    assert -1.35 < slope < -0.85, slope
    assert loads[0] > 3 * counts.mean()
