"""The whole delta layer (conv -> L2(q, k) -> recurrence -> gated norm), fp64 — TEST INFRASTRUCTURE.

Sources: model card "Agnes-3.0-Flash Preview", 架构 table, delta-rule row (kernel-4 causal conv
in front of the gated delta rule, a gated RMS-norm behind, fp32 state); discosf article
"Agnes 3.0 Flash 刚上线就刷屏…", section 二.1 (the layer runs as a chunked prefill and as a
stepwise decode).

Two plain compositions of the pinned single-step routines of this package, with nothing
rounded in between:
  * ``prefill_layer``: one sequence of T tokens in prefill mode;
  * ``decode_layer_step``: one token per batch entry, with the caches held in slots of a pool.
Reading where the pages are silent: the projection output x holds the channels q (Hk heads),
k (Hk heads), v (Hv heads) in that order; the conv covers all of them; only q and k are
L2-normalised.  Pinned in tests/test_oracle_pins.py: T decode steps equal one prefill of the
same T tokens, and the slot mapping only permutes the work.
"""
import numpy as np

from .conv import causal_conv
from .gdn import recurrence
from .norm import gated_rmsnorm
from .inputs import as_f64

D = 128


def _split(u, hk, hv):
    """[T, C] conv output -> q [T, Hk, D], k [T, Hk, D], v [T, Hv, D]."""
    T = u.shape[0]
    q = u[:, :hk * D].reshape(T, hk, D)
    k = u[:, hk * D:2 * hk * D].reshape(T, hk, D)
    v = u[:, 2 * hk * D:].reshape(T, hv, D)
    return q, k, v


def prefill_conv_recurrence(x, conv_w, cu_seqlens, conv_state, g, beta, initial_state, hk, hv,
                            conv_bias=None, scale=1.0, l2_eps=1e-6):
    """conv + SiLU + L2(q, k) -> recurrence over a packed batch, nothing rounded in between.

    x [T, C]; cu_seqlens [N+1]; conv_state [N, C, 3] or None (zeros); initial_state
    [N, Hv, D, D] or None.  Returns (o [T, Hv, D], final conv state [N, C, 3], final state).
    """
    u, cs1 = causal_conv(x, conv_w, cu_seqlens, conv_state, conv_bias, l2_heads=2 * hk, head_dim=D,
                         eps=l2_eps)
    q, k, v = _split(u, hk, hv)
    o, s1 = recurrence(q, k, v, g, beta, cu_seqlens, initial_state, scale)
    return o, cs1, s1


def prefill_layer(x, conv_w, conv_state, g, beta, z, norm_w, state, hk, hv, conv_bias=None,
                  scale=1.0, l2_eps=1e-6, norm_eps=1e-6):
    """One sequence of T tokens: x [T, C]; conv_state [C, 3] or None; state [Hv, D, D] or None.

    Returns (y [T, Hv, D], o [T, Hv, D], new conv state [C, 3], new state [Hv, D, D]).
    """
    x = as_f64(x)
    T = x.shape[0]
    cs = None if conv_state is None else as_f64(conv_state)[None]
    u, cs1 = causal_conv(x, conv_w, np.array([0, T]), cs, conv_bias, l2_heads=2 * hk, head_dim=D,
                         eps=l2_eps)
    q, k, v = _split(u, hk, hv)
    s0 = None if state is None else as_f64(state)[None]
    o, s1 = recurrence(q, k, v, g, beta, np.array([0, T]), s0, scale)
    y = gated_rmsnorm(o, z, norm_w, norm_eps)
    return y, o, cs1[0], s1[0]


def decode_layer_step(x, conv_w, conv_state, g, beta, z, norm_w, state, hk, hv, slots=None,
                      conv_bias=None, scale=1.0, l2_eps=1e-6, norm_eps=1e-6):
    """One token for each of B entries; caches in pools conv_state [S, C, 3], state [S, Hv, D, D].

    Entry b uses slot ``slots[b]`` (b when slots is None); an entry whose slot lies outside
    [0, S) is padding: its y and o rows are zero and no cache changes.  Returns
    (y [B, Hv, D], o [B, Hv, D], new conv_state pool, new state pool); the inputs are not modified.
    """
    x = as_f64(x)
    B = x.shape[0]
    cs_pool = np.array(as_f64(conv_state), copy=True)
    st_pool = np.array(as_f64(state), copy=True)
    S = cs_pool.shape[0]
    sl = np.arange(B) if slots is None else np.asarray(slots, np.int64)
    live = [b for b in range(B) if 0 <= sl[b] < S]
    y = np.zeros((B, hv, D))
    o = np.zeros((B, hv, D))
    if not live:
        return y, o, cs_pool, st_pool
    idx = np.array(live)
    u, cs1 = causal_conv(x[idx], conv_w, np.arange(len(idx) + 1), cs_pool[sl[idx]], conv_bias,
                         l2_heads=2 * hk, head_dim=D, eps=l2_eps)
    q, k, v = _split(u, hk, hv)
    ol, s1 = recurrence(q, k, v, as_f64(g)[idx], as_f64(beta)[idx], np.arange(len(idx) + 1),
                        st_pool[sl[idx]], scale)
    o[idx] = ol
    y[idx] = gated_rmsnorm(ol, as_f64(z)[idx], norm_w, norm_eps)
    cs_pool[sl[idx]] = cs1
    st_pool[sl[idx]] = s1
    return y, o, cs_pool, st_pool
