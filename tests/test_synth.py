"""Seeded input generators: determinism, shapes and distributions (CPU)."""
import hashlib

import numpy as np

from synth import (make_config, varlen_lengths, unit_vectors, gate_draws, LAYER,
                   decode_step_inputs, f32_to_bf16_bits, bf16_bits_to_f32)
from synth.configs import sequence_inputs


def _digest(d):
    h = hashlib.sha256()
    for key in sorted(d):
        val = d[key]
        if isinstance(val, np.ndarray):
            h.update(key.encode())
            h.update(val.tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    assert _digest(make_config(0)) == _digest(make_config(0))
    a = sequence_inputs(np.random.default_rng(5), [70, 3], 2, 6, 16, init="alternate")
    b = sequence_inputs(np.random.default_rng(5), [70, 3], 2, 6, 16, init="alternate")
    c = sequence_inputs(np.random.default_rng(6), [70, 3], 2, 6, 16, init="alternate")
    assert _digest(a) == _digest(b) != _digest(c)


def test_decode_step_inputs_seeded_per_step():
    a, b, c = decode_step_inputs(7, batch=4), decode_step_inputs(7, batch=4), decode_step_inputs(8, batch=4)
    assert _digest(a) == _digest(b) != _digest(c)
    assert a["q"].shape == (4, 16, 128) and a["v"].shape == (4, 48, 128)
    assert a["x"].shape == (4, LAYER["conv_channels"])


def test_config0_shapes_and_distributions():
    c = make_config(0)
    assert c["q"].dtype == np.float32 and c["q"].shape == (512, 1, 128)
    assert c["v"].shape == (512, 3, 128) and c["initial_state"] is None
    np.testing.assert_allclose(np.linalg.norm(c["k"].astype(np.float64), axis=-1), 1.0, rtol=1e-6)
    assert np.all((c["beta"] > 0) & (c["beta"] < 1)) and np.all(c["g"] < 0)
    # mean decay exp(g) for g = -softplus(N(0,1)) * 0.05 is about 0.96
    assert 0.95 < np.exp(c["g"]).mean() < 0.97


def test_varlen_lengths_recipe():
    L = varlen_lengths(np.random.default_rng(1004))
    assert len(L) == 32 and L.min() >= 512 and L.max() <= 32768
    assert 150_000 < L.sum() < 350_000


def test_bf16_inputs_are_rounded_unit_vectors():
    s = sequence_inputs(np.random.default_rng(3), [10], 2, 6, 128, dtype="bf16", init="normal")
    assert s["q"].dtype == np.uint16
    qf = bf16_bits_to_f32(s["q"]).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(qf, axis=-1), 1.0, atol=1e-2)
    assert s["initial_state"].shape == (1, 6, 128, 128)
    assert 0.009 < s["initial_state"].std() < 0.011


def test_bf16_roundtrip_and_rne_ties():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0); 1 + 3*2^-8 rounds up
    np.testing.assert_array_equal(bf16_bits_to_f32(f32_to_bf16_bits(x)),
                                  np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5], np.float32))


def test_gate_draws_ranges():
    g, b = gate_draws(np.random.default_rng(0), (1000, 4))
    assert np.all(g <= 0) and np.all((b > 0) & (b < 1))


def test_unit_vectors_norm():
    u = unit_vectors(np.random.default_rng(0), (50, 3, 128))
    np.testing.assert_allclose(np.linalg.norm(u.astype(np.float64), axis=-1), 1.0, rtol=1e-6)
