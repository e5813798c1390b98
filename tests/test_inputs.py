"""Seeded input generators: determinism, distributions, bf16 storage rounding."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_round_matches_torch_rne():
    """bf16 rounding is round-to-nearest-even, checked against torch's CPU conversion
    on ties, subnormals, signed zeros, infinities and random values."""
    edge = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 1.00390625, 1.01171875,
                     1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.0e38, 1e-40, -1e-40, 1.17549435e-38,
                     65504.0, 2 ** -133], dtype=np.float32)
    # exact ties: mantissa with the low 16 bits 0x8000, both parities of bit 16
    tie_bits = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00008000, 0x00018000], np.uint32)
    g = np.random.default_rng(0)
    vals = np.concatenate([edge, tie_bits.view(np.float32),
                           g.normal(size=10000).astype(np.float32),
                           (g.normal(size=1000) * 1e-39).astype(np.float32)])
    ours = W.bf16_round(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(W.bf16_round(np.array([np.nan], np.float32)))[0]


def test_bf16_bits_roundtrip():
    v = W.bf16_round(np.random.default_rng(1).normal(size=1000).astype(np.float32))
    np.testing.assert_array_equal(W.bf16_from_bits(W.bf16_bits(v)), v)


def test_generators_deterministic_and_keyed():
    a = W.prefill_inputs(W.C0, seed=0)
    b = W.prefill_inputs(W.C0, seed=0)
    c = W.prefill_inputs(W.C0, seed=1)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert not np.array_equal(a["x"], c["x"])
    assert not np.array_equal(a["x"], a["z"])  # separate streams per tensor


def test_c0_shapes_and_distributions():
    i = W.prefill_inputs(W.C0)
    assert i["x"].shape == (1, 32, 64) and i["Bm"].shape == (1, 32, 16)
    assert i["A_log"].shape == (64, 16) and i["conv_w"].shape == (64, 4)
    np.testing.assert_allclose(np.exp(i["A_log"][0]), np.arange(1, 17), rtol=1e-6)
    assert np.all(np.abs(i["conv_w"]) <= 0.5)
    assert not i["ssm_state"].any() and not i["conv_state"].any()
    big = W.prefill_inputs(W.C1)
    assert abs(big["x"].std() - 1.0) < 0.01 and abs(big["dt"].std() - 0.1) < 0.001
    assert np.all((big["dt0"] >= 1e-3) & (big["dt0"] <= 0.1))
    # the bias is the inverse softplus of dt0
    sp = np.logaddexp(0.0, big["dt_bias"].astype(np.float64))
    np.testing.assert_allclose(sp, big["dt0"], rtol=1e-5)


def test_bf16_workload_values_are_bf16():
    s = W.PrefillShape("t", B=1, T=16, D=32, io="bf16")
    i = W.prefill_inputs(s)
    for k in ("x", "z", "dt", "Bm", "Cm"):
        np.testing.assert_array_equal(W.bf16_round(i[k]), i[k])
    assert i["A_log"].dtype == np.float32  # parameters stay f32


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_config_table(name):
    s = W.CONFIGS[name]
    assert s.N == 16 and s.K == 4
    if name == "c3":
        assert (s.B, s.T, s.D, s.io) == (8, 4096, 5120, "bf16")
    if name == "c2":
        assert (s.L, s.B, s.D, s.steps) == (24, 64, 1536, 1000)


def test_store_large_path_equals_bf16_round():
    a = np.random.default_rng(3).normal(size=W._TORCH_ROUND_MIN + 17).astype(np.float32)
    np.testing.assert_array_equal(W.store(a, "bf16").view(np.uint32), W.bf16_round(a).view(np.uint32))
