"""Pins of the fp64 oracle against facts fixed by the mathematics, not by the oracle itself.

Every test here runs on the CPU.  Each names the property it pins and the
mistake it is there to catch.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from synth import unit_vectors, gate_draws


def _rand_inputs(rng, T, Hk, Hv, d, unit=True, g_scale=0.05):
    q = unit_vectors(rng, (T, Hk, d)).astype(np.float64) if unit else rng.standard_normal((T, Hk, d))
    k = unit_vectors(rng, (T, Hk, d)).astype(np.float64) if unit else rng.standard_normal((T, Hk, d))
    v = rng.standard_normal((T, Hv, d))
    g, beta = gate_draws(rng, (T, Hv), g_scale)
    return q, k, v, g.astype(np.float64), beta.astype(np.float64)


def _exact_unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- recurrence

def test_pin_beta_zero_is_pure_decay():
    """beta = 0: S_T = exp(sum g) S_0 and o_t = exp(gamma_t) S_0 q_t (decay placement, cumsum,
    output from the updated state)."""
    rng = np.random.default_rng(1)
    T, Hk, Hv, d = 37, 2, 6, 16
    q, k, v, g, beta = _rand_inputs(rng, T, Hk, Hv, d)
    beta[:] = 0.0
    S0 = rng.standard_normal((1, Hv, d, d))
    o, S = oracle.recurrence(q, k, v, g, beta, None, S0)
    gam = np.cumsum(g, axis=0)                     # [T, Hv]
    kh = np.arange(Hv) // 3
    exp_o = np.exp(gam)[:, :, None] * np.einsum("hij,thj->thi", S0[0], q[:, kh])
    np.testing.assert_allclose(o, exp_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S[0], np.exp(gam[-1])[:, None, None] * S0[0], rtol=1e-12)


def test_pin_orthonormal_retrieval():
    """alpha = 1, beta = 1, S_0 = 0, orthonormal keys: S_n = sum v_i k_i^T and S_n k_j = v_j
    (write semantics; a transposed state fails because S^T k_j != v_j)."""
    rng = np.random.default_rng(2)
    d, n = 32, 20
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm[:n]                                  # orthonormal rows
    k = keys[:, None, :]
    v = rng.standard_normal((n, 1, d))
    q = k.copy()
    g = np.zeros((n, 1))
    beta = np.ones((n, 1))
    o, S = oracle.recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(S[0, 0], v[:, 0].T @ keys, atol=1e-12)
    np.testing.assert_allclose(S[0, 0] @ keys.T, v[:, 0].T, atol=1e-12)
    # read-back after the last write still retrieves every stored pair
    np.testing.assert_allclose(o[-1, 0], v[-1, 0], atol=1e-12)


def test_pin_overwrite_any_gate_and_history():
    """beta = 1 with unit keys: S_t k_t = v_t for any decay and history, so q_t = k_t gives
    o_t = v_t (alpha multiplies the erase term too; o uses S_t, not S_{t-1})."""
    rng = np.random.default_rng(3)
    T, Hk, Hv, d = 25, 1, 3, 16
    k = _exact_unit(rng, (T, Hk, d))
    q = k.copy()
    v = rng.standard_normal((T, Hv, d))
    g = -rng.uniform(0.0, 2.0, (T, Hv))
    beta = np.ones((T, Hv))
    S0 = rng.standard_normal((1, Hv, d, d))
    o, _ = oracle.recurrence(q, k, v, g, beta, None, S0)
    np.testing.assert_allclose(o, v, atol=1e-12)


def test_pin_memoryless_limit():
    """g = -60 (alpha ~ 1e-26): o_t = beta_t (k_t . q_t) v_t."""
    rng = np.random.default_rng(4)
    T, Hk, Hv, d = 19, 2, 4, 8
    q, k, v, g, beta = _rand_inputs(rng, T, Hk, Hv, d, unit=False)
    g[:] = -60.0
    S0 = rng.standard_normal((1, Hv, d, d))
    o, _ = oracle.recurrence(q, k, v, g, beta, None, S0)
    kh = np.arange(Hv) // 2
    kq = np.einsum("thj,thj->th", k[:, kh], q[:, kh])
    np.testing.assert_allclose(o, beta[:, :, None] * kq[:, :, None] * v, rtol=1e-10, atol=1e-12)


def test_pin_gradient_step_on_regression_loss():
    """The delta-rule write is one gradient step of size beta on L(S) = 1/2 |S k - v|^2 taken from
    the decayed state alpha S_{t-1}.  The gradient is taken here by central finite differences,
    independently of the update formula (catches sign, transpose and missing-term mistakes)."""
    rng = np.random.default_rng(5)
    d = 6
    S0 = rng.standard_normal((d, d))
    k = rng.standard_normal(d)
    v = rng.standard_normal(d)
    q = rng.standard_normal(d)
    g, b = -0.3, 0.7
    Sp = np.exp(g) * S0
    loss = lambda S: 0.5 * np.sum((S @ k - v) ** 2)
    grad = np.zeros((d, d))
    h = 1e-5
    for i in range(d):
        for j in range(d):
            E = np.zeros((d, d))
            E[i, j] = h
            grad[i, j] = (loss(Sp + E) - loss(Sp - E)) / (2 * h)
    expected = Sp - b * grad
    o, S = oracle.recurrence(q[None, None], k[None, None], v[None, None],
                             np.array([[g]]), np.array([[b]]), None, S0[None, None])
    np.testing.assert_allclose(S[0, 0], expected, atol=1e-8)
    np.testing.assert_allclose(o[0, 0], expected @ q, atol=1e-8)


def test_pin_linearity_in_values_and_state():
    """(V, S_0) -> (O, S_T) is linear for fixed q, k, beta, g (catches stray constants)."""
    rng = np.random.default_rng(6)
    T, Hk, Hv, d = 21, 1, 2, 8
    q, k, v1, g, beta = _rand_inputs(rng, T, Hk, Hv, d)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, Hv, d, d))
    s2 = rng.standard_normal((1, Hv, d, d))
    a, b = 0.7, -1.3
    o1, f1 = oracle.recurrence(q, k, v1, g, beta, None, s1)
    o2, f2 = oracle.recurrence(q, k, v2, g, beta, None, s2)
    o3, f3 = oracle.recurrence(q, k, a * v1 + b * v2, g, beta, None, a * s1 + b * s2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-11)
    np.testing.assert_allclose(f3, a * f1 + b * f2, atol=1e-11)


@pytest.mark.parametrize("T1", [1, 63, 100])
def test_pin_split_invariance(T1):
    """prefill[0,T) == prefill[0,T1) -> state -> prefill[T1,T) (initial/final state plumbing)."""
    rng = np.random.default_rng(7)
    T, Hk, Hv, d = 160, 2, 6, 16
    q, k, v, g, beta = _rand_inputs(rng, T, Hk, Hv, d)
    S0 = rng.standard_normal((1, Hv, d, d)) * 0.1
    o, S = oracle.recurrence(q, k, v, g, beta, None, S0)
    oa, Sa = oracle.recurrence(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], None, S0)
    ob, Sb = oracle.recurrence(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], None, Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sb, S, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T", [1, 64, 100, 257])
def test_pin_matrix_form_equals_token_loop(T):
    """The whole-sequence closed form (a different derivation, solved with a dense library solve)
    equals the token loop to 1e-12 — the chunked prefill is exactly this re-association."""
    rng = np.random.default_rng(8 + T)
    Hk, Hv, d = 2, 6, 16
    q, k, v, g, beta = _rand_inputs(rng, T, Hk, Hv, d)
    S0 = rng.standard_normal((1, Hv, d, d)) * 0.1
    o1, S1 = oracle.recurrence(q, k, v, g, beta, None, S0, scale=0.5)
    o2, S2 = oracle.recurrence_matrix_form(q, k, v, g, beta, S0[0], scale=0.5)
    ref = np.abs(o1).max()
    assert np.abs(o1 - o2).max() <= 1e-12 * max(1.0, ref)
    assert np.abs(S1[0] - S2).max() <= 1e-12 * max(1.0, np.abs(S1).max())


def test_pin_head_mapping_contiguous_groups():
    """Value head h reads key head h // (Hv/Hk): with key head 1 silent (zero k and q) and
    S_0 = 0, value heads 3..5 stay exactly zero while 0..2 do not (an h % Hk mapping fails)."""
    rng = np.random.default_rng(9)
    T, Hk, Hv, d = 12, 2, 6, 8
    q, k, v, g, beta = _rand_inputs(rng, T, Hk, Hv, d)
    q[:, 1] = 0.0
    k[:, 1] = 0.0
    o, S = oracle.recurrence(q, k, v, g, beta)
    assert np.all(o[:, 3:] == 0.0) and np.all(S[0, 3:] == 0.0)
    assert np.all(np.abs(o[:, :3]).sum(axis=(0, 2)) > 0)


def test_pin_varlen_sequences_are_independent():
    """A packed batch equals each sequence run alone (no state leaks across cu_seqlens)."""
    rng = np.random.default_rng(10)
    lens = [5, 0, 17, 1, 64]
    T, Hk, Hv, d = sum(lens), 1, 3, 8
    q, k, v, g, beta = _rand_inputs(rng, T, Hk, Hv, d)
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0 = rng.standard_normal((len(lens), Hv, d, d))
    o, S = oracle.recurrence(q, k, v, g, beta, cu, S0)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, Sn = oracle.recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], None, S0[n:n + 1])
        np.testing.assert_array_equal(o[a:b], on)
        np.testing.assert_array_equal(S[n], Sn[0])
    np.testing.assert_array_equal(S[1], S0[1])     # empty sequence: state passes through


def test_pin_state_size_independent_of_length():
    """The final state's shape and byte size do not depend on T (model card, 架构: state size
    independent of sequence length)."""
    rng = np.random.default_rng(11)
    shapes = set()
    for T in (1, 64, 300):
        q, k, v, g, beta = _rand_inputs(rng, T, 1, 3, 8)
        _, S = oracle.recurrence(q, k, v, g, beta)
        shapes.add((S.shape, S.nbytes))
    assert len(shapes) == 1


def test_pin_scale_multiplies_output_only():
    rng = np.random.default_rng(12)
    q, k, v, g, beta = _rand_inputs(rng, 9, 1, 3, 8)
    o1, S1 = oracle.recurrence(q, k, v, g, beta, scale=1.0)
    o2, S2 = oracle.recurrence(q, k, v, g, beta, scale=0.25)
    np.testing.assert_allclose(o2, 0.25 * o1, rtol=1e-14)
    np.testing.assert_array_equal(S1, S2)


def test_pin_decode_step_iterated_equals_prefill():
    """Stepwise decode iterated over a sequence equals the whole-sequence closed form
    (the pages' two paths for one layer)."""
    rng = np.random.default_rng(13)
    T, Hk, Hv, d = 40, 2, 6, 8
    q, k, v, g, beta = _rand_inputs(rng, T, Hk, Hv, d)
    S0 = rng.standard_normal((1, Hv, d, d)) * 0.1
    o_ref, S_ref = oracle.recurrence_matrix_form(q, k, v, g, beta, S0[0])
    S = S0.copy()
    outs = []
    for t in range(T):
        ot, S = oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                   beta[t:t + 1], S)
        outs.append(ot[0])
    np.testing.assert_allclose(np.stack(outs), o_ref, atol=1e-12)
    np.testing.assert_allclose(S[0], S_ref, atol=1e-12)


def test_pin_heads_subset_matches_full():
    rng = np.random.default_rng(14)
    q, k, v, g, beta = _rand_inputs(rng, 20, 2, 6, 8)
    o, S = oracle.recurrence(q, k, v, g, beta)
    o2, S2 = oracle.recurrence(q, k, v, g, beta, heads=[1, 4])
    np.testing.assert_array_equal(o2[:, [1, 4]], o[:, [1, 4]])
    np.testing.assert_array_equal(S2[:, [1, 4]], S[:, [1, 4]])


# ---------------------------------------------------------------- conv

def _conv_library(x, w, hist):
    """Per-channel causal cross-correlation via numpy.correlate, SiLU via scipy's expit."""
    xh = np.concatenate([hist, x], axis=0)
    pre = np.stack([np.correlate(xh[:, c], w[c], mode="valid") for c in range(x.shape[1])], axis=1)
    return pre * expit(pre)


def test_pin_conv_equals_library_correlation():
    rng = np.random.default_rng(20)
    T, C, K = 30, 12, 4
    x = rng.standard_normal((T, C))
    w = rng.uniform(-0.5, 0.5, (C, K))
    st = rng.standard_normal((1, C, K - 1))
    y, fin = oracle.causal_conv(x, w, None, st)
    np.testing.assert_allclose(y, _conv_library(x, w, st[0].T), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(fin[0], x[-3:].T)


def test_pin_conv_current_tap_and_shift():
    """w = e_3 gives SiLU(x); w = e_0 gives a 3-token delay filled from the conv state."""
    rng = np.random.default_rng(21)
    T, C = 10, 5
    x = rng.standard_normal((T, C))
    st = rng.standard_normal((1, C, 3))
    w = np.zeros((C, 4))
    w[:, 3] = 1.0
    y, _ = oracle.causal_conv(x, w, None, st)
    np.testing.assert_allclose(y, x * expit(x), rtol=1e-13)
    w = np.zeros((C, 4))
    w[:, 0] = 1.0
    y, _ = oracle.causal_conv(x, w, None, st)
    delayed = np.concatenate([st[0].T, x[:-3]], axis=0)
    np.testing.assert_allclose(y, delayed * expit(delayed), rtol=1e-13)


def test_pin_conv_varlen_no_leak_and_short_sequences():
    rng = np.random.default_rng(22)
    lens = [1, 2, 0, 7, 3]
    C = 6
    x = rng.standard_normal((sum(lens), C))
    w = rng.uniform(-0.5, 0.5, (C, 4))
    st = rng.standard_normal((len(lens), C, 3))
    cu = np.concatenate([[0], np.cumsum(lens)])
    y, fin = oracle.causal_conv(x, w, cu, st)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        yn, fn = oracle.causal_conv(x[a:b], w, None, st[n:n + 1])
        np.testing.assert_array_equal(y[a:b], yn)
        np.testing.assert_array_equal(fin[n], fn[0])
        hist = np.concatenate([st[n].T, x[a:b]], axis=0)
        np.testing.assert_array_equal(fin[n], hist[-3:].T)


def test_pin_conv_split_with_state_handoff():
    rng = np.random.default_rng(23)
    T, C = 40, 4
    x = rng.standard_normal((T, C))
    w = rng.uniform(-0.5, 0.5, (C, 4))
    y, fin = oracle.causal_conv(x, w)
    ya, fa = oracle.causal_conv(x[:13], w)
    yb, fb = oracle.causal_conv(x[13:], w, None, fa)
    np.testing.assert_allclose(np.concatenate([ya, yb]), y, rtol=1e-14)
    np.testing.assert_array_equal(fb, fin)


def test_pin_conv_l2norm_of_leading_heads():
    rng = np.random.default_rng(24)
    T, d = 7, 8
    C = 4 * d
    x = rng.standard_normal((T, C))
    w = rng.uniform(-0.5, 0.5, (C, 4))
    y0, _ = oracle.causal_conv(x, w, l2_heads=0, head_dim=d)
    y2, _ = oracle.causal_conv(x, w, l2_heads=2, head_dim=d, eps=0.0)
    n = np.linalg.norm(y2[:, :2 * d].reshape(T, 2, d), axis=-1)
    np.testing.assert_allclose(n, 1.0, rtol=1e-13)
    # direction preserved, untouched heads unchanged
    np.testing.assert_allclose(y2[:, :d] * np.linalg.norm(y0[:, :d], axis=-1, keepdims=True),
                               y0[:, :d], rtol=1e-12)
    np.testing.assert_array_equal(y2[:, 2 * d:], y0[:, 2 * d:])


# ---------------------------------------------------------------- gated RMSNorm

def test_pin_norm_zero_gate_and_constant_rows():
    rng = np.random.default_rng(30)
    o = rng.standard_normal((5, 3, 16))
    w = rng.standard_normal(16)
    assert np.all(oracle.gated_rmsnorm(o, np.zeros_like(o), w) == 0.0)
    z = rng.standard_normal((5, 3, 16))
    c = -2.5
    y = oracle.gated_rmsnorm(np.full((5, 3, 16), c), z, w, eps=1e-6)
    exp = np.sign(c) * abs(c) / np.sqrt(c * c + 1e-6) * w * z * expit(z)
    np.testing.assert_allclose(y, exp, rtol=1e-13)


def test_pin_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(31)
    o = rng.standard_normal((40, 16))
    z = np.full_like(o, 50.0)                      # silu(50) = 50 to 1e-20
    y = oracle.gated_rmsnorm(o, z, np.ones(16), eps=0.0) / 50.0
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    y1 = oracle.gated_rmsnorm(o, z, np.ones(16), eps=0.0)
    y2 = oracle.gated_rmsnorm(7.0 * o, z, np.ones(16), eps=0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-12)


def test_oracle_upcast_of_bf16_patterns_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x7F80, 0x3E80], np.uint16)
    np.testing.assert_array_equal(oracle.as_f64(bits), [1.0, -1.0, 0.0, np.inf, 0.25])


# ---------------------------------------------------------------- whole layer

def _layer_inputs(rng, T, Hk, Hv, d=128):
    C = (2 * Hk + Hv) * d
    x = rng.standard_normal((T, C)) * 1.4
    w = rng.uniform(-0.5, 0.5, (C, 4))
    g, beta = gate_draws(rng, (T, Hv), 0.05)
    z = rng.standard_normal((T, Hv, d))
    nw = 1.0 + 0.1 * rng.standard_normal(d)
    return x, w, g.astype(np.float64), beta.astype(np.float64), z, nw


def test_pin_layer_decode_steps_equal_prefill():
    """T decode steps of the layer (conv history carried token to token, state carried in
    its slot) equal one prefill of the layer over the same T tokens: catches a wrong
    history shift, a history slot mix-up and a state hand-off error."""
    rng = np.random.default_rng(40)
    T, Hk, Hv = 12, 1, 3
    x, w, g, beta, z, nw = _layer_inputs(rng, T, Hk, Hv)
    C = x.shape[1]
    cs0 = rng.standard_normal((C, 3))
    s0 = rng.standard_normal((Hv, 128, 128)) * 0.01
    y_ref, o_ref, cs_ref, s_ref = oracle.prefill_layer(x, w, cs0, g, beta, z, nw, s0, Hk, Hv)
    # a pool of 3 slots, the sequence living in slot 2
    cs_pool = rng.standard_normal((3, C, 3))
    st_pool = rng.standard_normal((3, Hv, 128, 128))
    cs_pool[2], st_pool[2] = cs0, s0
    others = (cs_pool[:2].copy(), st_pool[:2].copy())
    for t in range(T):
        y, o, cs_pool, st_pool = oracle.decode_layer_step(
            x[t:t + 1], w, cs_pool, g[t:t + 1], beta[t:t + 1], z[t:t + 1], nw, st_pool, Hk, Hv,
            slots=[2])
        np.testing.assert_allclose(y[0], y_ref[t], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(o[0], o_ref[t], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(cs_pool[2], cs_ref, rtol=0, atol=0)
    np.testing.assert_allclose(st_pool[2], s_ref, rtol=1e-10, atol=1e-13)
    np.testing.assert_array_equal(cs_pool[:2], others[0])
    np.testing.assert_array_equal(st_pool[:2], others[1])


def test_pin_layer_channel_order_and_normalised_heads():
    """With the current-token tap only (w = [0, 0, 0, 1]) and one token from a zero state,
    S_1 = beta v k^T and o = beta (k . q) v with q, k the L2-normalised SiLU of the first and
    second 128-channel groups and v the SiLU of the third (not normalised); y is o's gated
    RMS-norm.  Catches a swapped q/k/v split or a normalised v."""
    rng = np.random.default_rng(41)
    Hk, Hv, d = 1, 1, 128
    x = rng.standard_normal((1, 3 * d))
    w = np.zeros((3 * d, 4))
    w[:, 3] = 1.0
    g = np.array([[-0.3]])
    beta = np.array([[0.7]])
    z = rng.standard_normal((1, Hv, d))
    nw = 1.0 + 0.1 * rng.standard_normal(d)
    y, o, _, S = oracle.prefill_layer(x, w, None, g, beta, z, nw, None, Hk, Hv)
    act = x[0] * expit(x[0])
    q = act[:d] / np.sqrt(act[:d] @ act[:d] + 1e-6)
    k = act[d:2 * d] / np.sqrt(act[d:2 * d] @ act[d:2 * d] + 1e-6)
    v = act[2 * d:]
    np.testing.assert_allclose(S[0], 0.7 * np.outer(v, k), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], 0.7 * (k @ q) * v, rtol=1e-12, atol=1e-15)
    rms = np.sqrt(np.mean(o[0, 0] ** 2) + 1e-6)
    np.testing.assert_allclose(y[0, 0], o[0, 0] / rms * nw * z[0, 0] * expit(z[0, 0]), rtol=1e-12)


def test_pin_layer_slots_permute_and_padding_is_inert():
    """Entries mapped to permuted slots give the rows of the identity mapping on a permuted
    pool; a padding entry (slot -1 or beyond the pool) yields zero rows and changes nothing."""
    rng = np.random.default_rng(42)
    B, Hk, Hv, S = 4, 1, 2, 6
    x, w, g, beta, z, nw = _layer_inputs(rng, B, Hk, Hv)
    C = x.shape[1]
    cs = rng.standard_normal((S, C, 3))
    st = rng.standard_normal((S, Hv, 128, 128)) * 0.01
    slots = np.array([4, -1, 0, 7])  # entries 1 and 3 are padding
    y, o, cs1, st1 = oracle.decode_layer_step(x, w, cs, g, beta, z, nw, st, Hk, Hv, slots=slots)
    live = [0, 2]
    y2, o2, cs2, st2 = oracle.decode_layer_step(x[live], w, cs[slots[live]], g[live], beta[live], z[live],
                                                nw, st[slots[live]], Hk, Hv)
    np.testing.assert_array_equal(y[live], y2)
    np.testing.assert_array_equal(o[live], o2)
    np.testing.assert_array_equal(cs1[slots[live]], cs2)
    np.testing.assert_array_equal(st1[slots[live]], st2)
    assert not y[[1, 3]].any() and not o[[1, 3]].any()
    untouched = [1, 2, 3, 5]
    np.testing.assert_array_equal(cs1[untouched], cs[untouched])
    np.testing.assert_array_equal(st1[untouched], st[untouched])


def test_pin_packed_layer_prefill_equals_per_sequence():
    """The packed conv + recurrence over several sequences (with histories and initial states)
    equals the single-sequence layer run on each: no history, state or conv tap crosses a
    sequence boundary, and each sequence's final history and state land in its own slot."""
    rng = np.random.default_rng(43)
    Hk, Hv = 1, 2
    lens = [5, 0, 2, 9]
    T = sum(lens)
    x, w, g, beta, z, nw = _layer_inputs(rng, T, Hk, Hv)
    C = x.shape[1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    cs = rng.standard_normal((len(lens), C, 3))
    s0 = rng.standard_normal((len(lens), Hv, 128, 128)) * 0.01
    o, cs1, s1 = oracle.prefill_conv_recurrence(x, w, cu, cs, g, beta, s0, Hk, Hv)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        if b == a:
            np.testing.assert_array_equal(cs1[n], cs[n])
            np.testing.assert_array_equal(s1[n], s0[n])
            continue
        _, on, csn, sn = oracle.prefill_layer(x[a:b], w, cs[n], g[a:b], beta[a:b], z[a:b], nw, s0[n], Hk, Hv)
        np.testing.assert_allclose(o[a:b], on, rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(cs1[n], csn)
        np.testing.assert_allclose(s1[n], sn, rtol=1e-12, atol=1e-14)
