"""Pins of the fp64 attention oracle against facts fixed by the mathematics and the pages, not by
the oracle itself.  CPU only; each test names the mistake it is there to catch.
"""
import math

import numpy as np

import oracle

D = 256


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_pin_attention_brute_force_loops():
    """Scores, causal mask, 1/sqrt(256) scale, softmax and the GQA head map, recomputed with
    scalar loops over two packed sequences (mask direction, off-by-one in the prefix, a
    transposed operand, a wrong scale or head map fail here)."""
    rng = np.random.default_rng(7)
    hq, hkv = 4, 2
    lens = [3, 4]
    cu = np.array([0, 3, 7])
    T = 7
    q, k, v = _rand(rng, T, hq, D), _rand(rng, T, hkv, D), _rand(rng, T, hkv, D)
    got = oracle.causal_attention(q, k, v, cu)
    for n in range(2):
        a = cu[n]
        for t in range(lens[n]):
            for h in range(hq):
                g = h // 2
                sc = []
                for j in range(t + 1):
                    sc.append(sum(q[a + t, h, i] * k[a + j, g, i] for i in range(D)) / 16.0)
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                z = sum(e)
                want = [sum(e[j] / z * v[a + j, g, i] for j in range(t + 1)) for i in range(0, D, 37)]
                np.testing.assert_allclose(got[a + t, h, ::37], want, rtol=1e-12, atol=1e-13)


def test_pin_identical_keys_average_the_prefix():
    """Equal keys make the softmax uniform over the causal prefix: output t is the mean of
    v[0..t] (inclusive prefix, normalisation)."""
    rng = np.random.default_rng(8)
    T = 9
    q = _rand(rng, T, 1, D)
    k = np.tile(_rand(rng, 1, 1, D), (T, 1, 1))
    v = _rand(rng, T, 1, D)
    got = oracle.causal_attention(q, k, v, [0, T])
    want = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None, None]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_pin_gate_and_first_token():
    """A sequence's first token attends only to itself: o = v * sigmoid(gate), whatever q and k;
    gate 0 halves it (sigmoid, not SiLU or tanh)."""
    rng = np.random.default_rng(9)
    q, k, v, gate = _rand(rng, 1, 6, D), _rand(rng, 1, 1, D), _rand(rng, 1, 1, D), _rand(rng, 1, 6, D)
    w = np.ones(D)
    o, _ = oracle.attention_prefill(q, k, v, gate, [0, 1], w, w)
    np.testing.assert_allclose(o[0], v[0, 0][None, :] / (1 + np.exp(-gate[0])), rtol=1e-13)
    o0, _ = oracle.attention_prefill(q, k, v, np.zeros_like(gate), [0, 1], w, w)
    np.testing.assert_allclose(o0[0], 0.5 * np.tile(v[0], (6, 1)), rtol=1e-13)


def test_pin_rms_norm_closed_form():
    """Constant rows c: the norm gives sign(c) |c| / sqrt(c^2 + eps) times the weight (mean of
    squares, not sum; eps inside the root; weight multiplied)."""
    w = np.linspace(0.5, 1.5, D)
    for c in (3.0, -0.25, 1e-4):
        got = oracle.rms_norm_heads(np.full((1, D), c), w, 1e-6)
        np.testing.assert_allclose(got[0], np.sign(c) * abs(c) / math.sqrt(c * c + 1e-6) * w, rtol=1e-13)


def test_pin_rotary_pair_closed_form():
    """A unit vector on dim j at position p turns to cos / sin of p * 1e7^(-j/32) on dims j and
    j + 32 (pairing j with j + 32, base 1e7, rotary span 64)."""
    for j, p in [(0, 5), (1, 7), (31, 1000), (17, 12345)]:
        x = np.zeros((1, 1, D))
        x[0, 0, j] = 1.0
        theta = p * (1e7 ** (-j / 32.0))
        got = oracle.apply_rotary(x, oracle.rope_angles(np.full((3, 1), p)))
        want = np.zeros(D)
        want[j] = math.cos(theta)
        want[j + 32] = math.sin(theta)
        np.testing.assert_allclose(got[0, 0], want, atol=1e-12)


def test_pin_rotary_relative_position_and_untouched_tail():
    """q and k turned at text positions m and n meet in a dot product that depends only on
    m - n (same direction of turn for both); dims 64..255 never change."""
    rng = np.random.default_rng(10)
    q, k = _rand(rng, 1, 1, D), _rand(rng, 1, 1, D)

    def dot(m, n):
        qr = oracle.apply_rotary(q, oracle.rope_angles(np.full((3, 1), m)))
        kr = oracle.apply_rotary(k, oracle.rope_angles(np.full((3, 1), n)))
        return float((qr * kr).sum()), qr
    a, qr = dot(20, 3)
    b, _ = dot(117, 100)
    assert abs(a - b) < 1e-9 * max(1.0, abs(a))
    np.testing.assert_array_equal(qr[0, 0, 64:], q[0, 0, 64:])


def test_pin_mrope_axis_interleave_11_11_10():
    """Frequency j follows axis j mod 3 (text, height, width): moving one axis turns exactly the
    pairs of its frequencies, 11, 11 and 10 of them."""
    rng = np.random.default_rng(11)
    x = _rand(rng, 1, 1, D)
    base = oracle.apply_rotary(x, oracle.rope_angles(np.zeros((3, 1))))
    counts = []
    for axis in range(3):
        pos = np.zeros((3, 1))
        pos[axis] = 1e5  # turns even the slowest frequency (1e7^(-31/32)) by ~0.016 rad
        y = oracle.apply_rotary(x, oracle.rope_angles(pos))
        moved = [j for j in range(32) if np.abs(y[0, 0, [j, j + 32]] - base[0, 0, [j, j + 32]]).max() > 1e-9]
        assert moved == [j for j in range(32) if j % 3 == axis]
        counts.append(len(moved))
    assert counts == [11, 11, 10]


def test_pin_gqa_equals_repeated_kv_heads():
    """Six query heads on one KV head equal six query heads on six copies of it (contiguous
    groups: query head h reads KV head h // 6)."""
    rng = np.random.default_rng(12)
    T = 6
    q, k, v = _rand(rng, T, 12, D), _rand(rng, T, 2, D), _rand(rng, T, 2, D)
    a = oracle.causal_attention(q, k, v, [0, T])
    b = oracle.causal_attention(q, np.repeat(k, 6, axis=1), np.repeat(v, 6, axis=1), [0, T])
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_pin_decode_steps_equal_prefill():
    """Decoding a sequence token by token from an empty cache gives the prefill's rows, and the
    cache ends up holding the prefill's normalised, rotated k and the raw v (cache layout,
    positions of decoded tokens, norm and rotary of the new token)."""
    rng = np.random.default_rng(13)
    T, hq, hkv = 5, 6, 1
    q, k, v, gate = _rand(rng, T, hq, D), _rand(rng, T, hkv, D), _rand(rng, T, hkv, D), _rand(rng, T, hq, D)
    qw, kw = 1 + 0.1 * _rand(rng, D), 1 + 0.1 * _rand(rng, D)
    o, kr = oracle.attention_prefill(q, k, v, gate, [0, T], qw, kw)
    kc = np.zeros((1, T, hkv, D))
    vc = np.zeros((1, T, hkv, D))
    for t in range(T):
        ot, kc, vc = oracle.attention_decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], gate[t:t + 1], kc, vc, [t], qw, kw)
        np.testing.assert_allclose(ot[0], o[t], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(kc[0], kr, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(vc[0], v)


def test_pin_packed_sequences_are_independent():
    """A packed batch equals each sequence run alone (no key crosses a cu_seqlens boundary;
    positions restart at each sequence)."""
    rng = np.random.default_rng(14)
    lens = [4, 0, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = sum(lens)
    q, k, v, gate = _rand(rng, T, 6, D), _rand(rng, T, 1, D), _rand(rng, T, 1, D), _rand(rng, T, 6, D)
    w = np.ones(D)
    o, kr = oracle.attention_prefill(q, k, v, gate, cu, w, w)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        if b > a:
            on, kn = oracle.attention_prefill(q[a:b], k[a:b], v[a:b], gate[a:b], [0, b - a], w, w)
            np.testing.assert_allclose(o[a:b], on, rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(kr[a:b], kn, rtol=1e-13, atol=1e-14)


def test_pin_row_subset_equals_full_attention():
    """The per-row routine used for large checks gives the full routine's rows (sequence start
    found from cu_seqlens, head map, causal prefix)."""
    rng = np.random.default_rng(15)
    cu = np.array([0, 5, 5, 12])
    q, k, v = _rand(rng, 12, 6, D), _rand(rng, 12, 2, D), _rand(rng, 12, 2, D)
    full = oracle.causal_attention(q, k, v, cu)
    rows, heads = [0, 4, 5, 6, 11], [0, 2, 3, 5]
    sub = oracle.causal_attention_rows(q, k, v, cu, rows, heads)
    np.testing.assert_allclose(sub, full[rows][:, heads], rtol=1e-13, atol=1e-14)
