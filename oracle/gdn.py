"""Gated delta-rule recurrence, fp64, token by token (the stepwise definition).

Sources:
  * model card "Agnes-3.0-Flash Preview", 架构 table, delta-rule row: 16 key /
    48 value heads, head dim 128, fp32 recurrent state;
  * discosf article "Agnes 3.0 Flash 刚上线就刷屏…", section 二.1: a chunked
    prefill (chunk 64) and a stepwise decode compute the same layer;
  * Yang, Kautz & Hatamizadeh, "Gated Delta Networks" (ICLR 2025), the gated
    delta rule: S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t.

Readings where the pages are silent:
  * gate: a_t = exp(g_t) with g a per-(token, value head) log-decay;
  * head mapping: value head h reads key head floor(h / (Hv / Hk)) for both q
    and k (contiguous groups of Hv/Hk value heads per key head);
  * state orientation: S[h] is [d_v, d_k] (rows = value dim), the shape of v k^T;
  * output uses the updated state S_t; an optional output scale multiplies o
    (1.0 = the formula as written);
  * sequences in a packed batch are independent; each starts from its own
    initial state (zeros when none is given).
"""
import numpy as np

from .inputs import as_f64


def key_head_of(num_k_heads, num_v_heads):
    """Key head index read by each value head (contiguous groups)."""
    if num_v_heads % num_k_heads:
        raise ValueError("value heads must be a multiple of key heads")
    return np.arange(num_v_heads) // (num_v_heads // num_k_heads)


def recurrence(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=1.0,
               heads=None):
    """Token-by-token gated delta rule over a packed batch.

    q, k: [T, Hk, dk]; v: [T, Hv, dv]; g, beta: [T, Hv]; cu_seqlens: [N+1]
    (None = one sequence); initial_state: [N, Hv, dv, dk] or None (zeros).
    ``heads``: optional list of value heads to evaluate (others are skipped and
    returned as zeros) so that large workloads can be checked on a subset.
    Returns (o [T, Hv, dv], final_state [N, Hv, dv, dk]) in fp64.
    """
    q, k, v, g, beta = (as_f64(a) for a in (q, k, v, g, beta))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, np.int64)
    N = len(cu) - 1
    hs = np.arange(Hv) if heads is None else np.asarray(heads)
    kh = key_head_of(Hk, Hv)[hs]
    o = np.zeros((T, Hv, dv))
    final = np.zeros((N, Hv, dv, dk))
    S0 = None if initial_state is None else as_f64(initial_state)
    for n in range(N):
        if S0 is None:
            S = np.zeros((len(hs), dv, dk))
        else:
            S = S0[n][hs].copy()
        for t in range(int(cu[n]), int(cu[n + 1])):
            a = np.exp(g[t, hs])[:, None, None]        # alpha_t per head
            b = beta[t, hs][:, None, None]             # beta_t per head
            kt = k[t, kh]                              # [H, dk]
            qt = q[t, kh]
            vt = v[t, hs]                              # [H, dv]
            Sk = np.einsum("hij,hj->hi", S, kt)        # S_{t-1} k_t
            # a S (I - b k k^T) + b v k^T, expanded by the rank-one structure
            S = (a * S
                 - a * b * np.einsum("hi,hj->hij", Sk, kt)
                 + b * np.einsum("hi,hj->hij", vt, kt))
            o[t, hs] = scale * np.einsum("hij,hj->hi", S, qt)
        final[n, hs] = S
    return o, final


def decode_step(q, k, v, g, beta, state, scale=1.0, heads=None):
    """One stepwise decode token for each of B independent sequences.

    q, k: [B, Hk, dk]; v: [B, Hv, dv]; g, beta: [B, Hv]; state: [B, Hv, dv, dk].
    Returns (o [B, Hv, dv], new_state) — the recurrence applied to a length-1
    sequence per batch entry.
    """
    B = np.asarray(q).shape[0]
    cu = np.arange(B + 1)
    return recurrence(q, k, v, g, beta, cu, state, scale, heads)


def recurrence_matrix_form(q, k, v, g, beta, initial_state=None, scale=1.0):
    """Whole-sequence closed form of the same recurrence (one sequence, all heads).

    Used only to pin the token loop.  With Gamma_t = sum_{s<=t} g_s and
    D[t, s] = exp(Gamma_t - Gamma_s) for s <= t (0 above the diagonal), unroll
    S_t = exp(Gamma_t) S_0 + sum_{s<=t} D[t, s] u_s k_s^T.  The pseudo-values u
    solve (I + A) U = diag(beta) (V - diag(exp Gamma) K S_0^T) with
    A = strictly_lower(diag(beta) (D * K K^T)); then
    O = diag(exp Gamma) Q S_0^T + (D * Q K^T) U and
    S_T = exp(Gamma_T) S_0 + (diag(exp(Gamma_T - Gamma)) U)^T K.
    A dense linear solve (numpy) is the only library step.
    """
    q, k, v, g, beta = (as_f64(a) for a in (q, k, v, g, beta))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    kh = key_head_of(Hk, Hv)
    o = np.zeros((T, Hv, dv))
    final = np.zeros((Hv, dv, dk))
    for h in range(Hv):
        Q, K, V = q[:, kh[h]], k[:, kh[h]], v[:, h]
        S0 = np.zeros((dv, dk)) if initial_state is None else as_f64(initial_state)[h]
        Gam = np.cumsum(g[:, h])
        D = np.tril(np.exp(Gam[:, None] - Gam[None, :]))
        A = np.tril(beta[:, h][:, None] * D * (K @ K.T), k=-1)
        rhs = beta[:, h][:, None] * (V - np.exp(Gam)[:, None] * (K @ S0.T))
        U = np.linalg.solve(np.eye(T) + A, rhs)
        o[:, h] = scale * (np.exp(Gam)[:, None] * (Q @ S0.T) + (D * (Q @ K.T)) @ U)
        final[h] = np.exp(Gam[-1]) * S0 + (np.exp(Gam[-1] - Gam)[:, None] * U).T @ K
    return o, final
