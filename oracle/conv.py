"""Depth-wise causal convolution (kernel 4) + SiLU, and per-head L2 normalisation, fp64.

Sources: model card "Agnes-3.0-Flash Preview", 架构 table, delta-rule row (a
causal convolution of kernel 4 in front of the recurrence); discosf article
"Agnes 3.0 Flash 刚上线就刷屏…", section 二.1 (the same kernel-4 causal conv).

Readings where the pages are silent:
  * depth-wise: each channel c has its own taps w[c, 0..K-1];
  * causal cross-correlation with K-1 = 3 tokens of left context:
      y[t, c] = SiLU(bias[c] + sum_{j=0}^{K-1} w[c, j] * x_hat[t - (K-1) + j, c]),
    so w[c, K-1] multiplies the current token;
  * x_hat before a sequence's first token comes from that sequence's conv state
    [C, K-1] (oldest first), or zeros when none is given; nothing crosses a
    sequence boundary of a packed batch;
  * the returned conv state is the last K-1 values of x_hat (oldest first);
  * SiLU(u) = u / (1 + exp(-u));
  * the L2 normalisation divides each of the leading ``l2_heads`` heads of
    ``head_dim`` channels by sqrt(sum of squares + eps), after the SiLU.
"""
import numpy as np

from .inputs import as_f64


def silu(u):
    """u * sigmoid(u) = u / (1 + exp(-u))."""
    return u / (1.0 + np.exp(-u))


def l2norm_heads(y, l2_heads, head_dim, eps):
    """Divide each of the first ``l2_heads`` channel groups of ``head_dim`` by its L2 norm."""
    y = np.array(y, dtype=np.float64, copy=True)
    if l2_heads:
        n = l2_heads * head_dim
        blk = y[:, :n].reshape(y.shape[0], l2_heads, head_dim)
        blk = blk / np.sqrt((blk * blk).sum(axis=-1, keepdims=True) + eps)
        y[:, :n] = blk.reshape(y.shape[0], n)
    return y


def causal_conv(x, w, cu_seqlens=None, conv_state=None, bias=None, l2_heads=0,
                head_dim=128, eps=1e-6):
    """Causal depth-wise conv + SiLU (+ L2 norm of leading heads) over a packed batch.

    x: [T, C]; w: [C, K]; cu_seqlens: [N+1] (None = one sequence); conv_state:
    [N, C, K-1] oldest first, or None (zeros); bias: [C] or None.
    Decode mode is the special case cu_seqlens = 0..N (one token per sequence).
    Returns (y [T, C], final_state [N, C, K-1]) in fp64.
    """
    x = as_f64(x)
    w = as_f64(w)
    T, C = x.shape
    K = w.shape[1]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, np.int64)
    N = len(cu) - 1
    b = np.zeros(C) if bias is None else as_f64(bias)
    y = np.zeros((T, C))
    final = np.zeros((N, C, K - 1))
    for n in range(N):
        hist = np.zeros((K - 1, C)) if conv_state is None else as_f64(conv_state)[n].T
        seg = np.concatenate([hist, x[int(cu[n]):int(cu[n + 1])]], axis=0)  # x_hat from t-(K-1)
        L = seg.shape[0] - (K - 1)
        acc = np.tile(b, (L, 1))
        for j in range(K):
            acc += w[:, j][None, :] * seg[j:j + L]
        y[int(cu[n]):int(cu[n + 1])] = silu(acc)
        final[n] = seg[-(K - 1):].T
    y = l2norm_heads(y, l2_heads, head_dim, eps)
    return y, final
