"""Workload recipes for the gated delta-rule layer (seeded, synthetic).

Shapes follow the layer the model card describes ("Agnes-3.0-Flash Preview",
section 架构, delta-rule row): 16 key heads, 48 value heads, head dim 128,
kernel-4 causal conv over the fused q|k|v channels, hidden size 5120.

Distributions (one recipe for every workload):
  * q, k: standard normal vectors scaled to unit length per head (a random
    direction on the sphere), then stored in the workload's dtype;
  * v: standard normal;
  * beta = sigmoid(N(0, 1)); log-decay g = -softplus(N(0, 1)) * 0.05,
    one value per (token, value head);
  * initial states: zeros or N(0, 0.01^2) (0.01 is a standard deviation).

numpy's PCG64 ``default_rng`` is the only source of randomness; every
workload derives its seed from ``1000 + index`` so the same bytes are
produced on any host.
"""
import numpy as np

from .bf16 import f32_to_bf16_bits

# Layer geometry (model card, 架构 table; discosf article, section 二.1).
LAYER = dict(
    num_k_heads=16,
    num_v_heads=48,
    head_dim=128,
    hidden=5120,
    conv_kernel=4,
    conv_channels=2 * 16 * 128 + 48 * 128,  # q | k | v = 10240
    chunk=64,
)

# Standard deviation of one projection output when N(0,1) activations meet
# N(0, 0.02^2) weights over 5120 inputs: sqrt(5120) * 0.02.
PROJ_STD = float(np.sqrt(5120.0) * 0.02)

_BLOCK = 8192  # tokens generated per draw, bounds host memory for long inputs


def unit_vectors(rng, shape):
    """Random directions: N(0,1) samples scaled to unit L2 norm on the last axis (fp32)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    n = np.sqrt(np.square(x, dtype=np.float64).sum(axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def gate_draws(rng, shape, g_scale=0.05):
    """(g, beta): g = -softplus(N(0,1)) * g_scale, beta = sigmoid(N(0,1)); fp32."""
    a = rng.standard_normal(shape)
    b = rng.standard_normal(shape)
    beta = 1.0 / (1.0 + np.exp(-a))
    g = -np.logaddexp(0.0, b) * g_scale
    return g.astype(np.float32), beta.astype(np.float32)


def _store(x, dtype):
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def varlen_lengths(rng, count=32, lo=512, hi=32768):
    """Log-uniform integer lengths on [lo, hi]."""
    u = rng.uniform(np.log(lo), np.log(hi), size=count)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)


def sequence_inputs(rng, lengths, num_k_heads, num_v_heads, head_dim, dtype="bf16",
                    init=None, init_std=0.01, g_scale=0.05):
    """Packed varlen inputs for the recurrence.

    ``init``: None (no initial state), "normal" (all sequences N(0, init_std^2)),
    "alternate" (even sequences zero, odd ones normal) or "zeros".
    Returns a dict of numpy arrays; q/k/v are uint16 bf16 patterns when
    ``dtype == "bf16"`` and float32 otherwise.
    """
    lengths = [int(x) for x in lengths]
    total = int(sum(lengths))
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    st = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((total, num_k_heads, head_dim), st)
    k = np.empty((total, num_k_heads, head_dim), st)
    v = np.empty((total, num_v_heads, head_dim), st)
    g = np.empty((total, num_v_heads), np.float32)
    beta = np.empty((total, num_v_heads), np.float32)
    for t0 in range(0, total, _BLOCK):
        t1 = min(total, t0 + _BLOCK)
        n = t1 - t0
        q[t0:t1] = _store(unit_vectors(rng, (n, num_k_heads, head_dim)), dtype)
        k[t0:t1] = _store(unit_vectors(rng, (n, num_k_heads, head_dim)), dtype)
        v[t0:t1] = _store(rng.standard_normal((n, num_v_heads, head_dim), dtype=np.float32), dtype)
        g[t0:t1], beta[t0:t1] = gate_draws(rng, (n, num_v_heads), g_scale)
    n_seq = len(lengths)
    s0 = None
    if init is not None:
        s0 = np.zeros((n_seq, num_v_heads, head_dim, head_dim), np.float32)
        for i in range(n_seq):
            if init == "normal" or (init == "alternate" and i % 2 == 1):
                s0[i] = rng.standard_normal((num_v_heads, head_dim, head_dim),
                                            dtype=np.float32) * np.float32(init_std)
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu, initial_state=s0,
                dtype=dtype, num_k_heads=num_k_heads, num_v_heads=num_v_heads,
                head_dim=head_dim)


def layer_prefill_inputs(rng, T, dtype="bf16"):
    """Full-layer prefill inputs: raw q|k|v projection outputs, conv and norm parameters.

    x = N(0,1)[T, 5120] @ N(0, 0.02^2)[5120, 10240], computed in fp32 on the host
    and rounded to bf16 (this projection only generates data).  Conv weights are
    U(-1/2, 1/2) (the 1/sqrt(fan_in) bound for fan-in 4), no bias, zero conv history;
    the norm weight is 1 + 0.1 N(0,1); the gate z is N(0,1).
    """
    L = LAYER
    C = L["conv_channels"]
    xs = rng.standard_normal((T, L["hidden"]), dtype=np.float32)
    wp = rng.standard_normal((L["hidden"], C), dtype=np.float32) * np.float32(0.02)
    x = xs @ wp
    del xs, wp
    conv_w = rng.uniform(-0.5, 0.5, size=(C, L["conv_kernel"])).astype(np.float32)
    g, beta = gate_draws(rng, (T, L["num_v_heads"]))
    z = rng.standard_normal((T, L["num_v_heads"], L["head_dim"]), dtype=np.float32)
    norm_w = (1.0 + 0.1 * rng.standard_normal(L["head_dim"])).astype(np.float32)
    return dict(x=_store(x, dtype), conv_w=_store(conv_w, dtype), g=g, beta=beta,
                z=_store(z, dtype), norm_w=_store(norm_w, dtype),
                cu_seqlens=np.array([0, T], np.int32), dtype=dtype, **L)


def layer_sequence_inputs(rng, lengths, init=None, init_std=0.01, g_scale=0.05):
    """Whole-layer prefill inputs over a packed batch of ``lengths`` tokens, with the raw
    projection output x drawn directly from its distribution N(0, PROJ_STD^2) (the projection
    matmul of ``layer_prefill_inputs`` is too costly on the host at 65536 tokens and beyond).

    Conv weights U(-1/2, 1/2), no bias, zero conv history; g, beta as every workload; z N(0,1);
    norm weight 1 + 0.1 N(0,1); initial states per ``init`` as in ``sequence_inputs``.  x and z
    are drawn in blocks of tokens, so host memory stays near the size of the stored arrays.
    """
    L = LAYER
    lengths = [int(n) for n in lengths]
    total = int(sum(lengths))
    C, hv, D = L["conv_channels"], L["num_v_heads"], L["head_dim"]
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    conv_w = f32_to_bf16_bits(rng.uniform(-0.5, 0.5, size=(C, L["conv_kernel"])).astype(np.float32))
    norm_w = f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    x = np.empty((total, C), np.uint16)
    z = np.empty((total, hv, D), np.uint16)
    g = np.empty((total, hv), np.float32)
    beta = np.empty((total, hv), np.float32)
    for t0 in range(0, total, _BLOCK):
        t1 = min(total, t0 + _BLOCK)
        n = t1 - t0
        x[t0:t1] = f32_to_bf16_bits(rng.standard_normal((n, C), dtype=np.float32) * np.float32(PROJ_STD))
        z[t0:t1] = f32_to_bf16_bits(rng.standard_normal((n, hv, D), dtype=np.float32))
        g[t0:t1], beta[t0:t1] = gate_draws(rng, (n, hv), g_scale)
    s0 = None
    if init is not None:
        s0 = np.zeros((len(lengths), hv, D, D), np.float32)
        for i in range(len(lengths)):
            if init == "normal" or (init == "alternate" and i % 2 == 1):
                s0[i] = rng.standard_normal((hv, D, D), dtype=np.float32) * np.float32(init_std)
    return dict(x=x, conv_w=conv_w, g=g, beta=beta, z=z, norm_w=norm_w, cu_seqlens=cu,
                initial_state=s0, dtype="bf16", **L)


def make_layer_config(index):
    """Whole-layer (conv -> recurrence -> gated norm) inputs for the long and the varlen
    workloads, seeded with [1000 + index, 1]: 2 = one sequence of 65536 tokens with an initial
    state N(0, 0.01^2); 4 = the 32 log-uniform lengths of workload 4 (the same lengths), initial
    states zero for even and N(0, 0.01^2) for odd sequences."""
    if index == 2:
        return layer_sequence_inputs(np.random.default_rng([1002, 1]), [65536], init="normal")
    if index == 4:
        lengths = varlen_lengths(np.random.default_rng(1004))
        return layer_sequence_inputs(np.random.default_rng([1004, 1]), lengths, init="alternate")
    raise ValueError(f"no whole-layer variant of workload {index}")


def decode_state_inputs(rng, batch):
    """Decode workload state: fp32 states N(0, 0.01^2), bf16 conv cache, conv weights."""
    L = LAYER
    state = np.empty((batch, L["num_v_heads"], L["head_dim"], L["head_dim"]), np.float32)
    for b in range(batch):
        state[b] = rng.standard_normal(state.shape[1:], dtype=np.float32) * np.float32(0.01)
    conv_cache = f32_to_bf16_bits(
        rng.standard_normal((batch, L["conv_channels"], L["conv_kernel"] - 1),
                            dtype=np.float32) * np.float32(PROJ_STD))
    conv_w = f32_to_bf16_bits(
        rng.uniform(-0.5, 0.5, size=(L["conv_channels"], L["conv_kernel"])).astype(np.float32))
    # gated-norm weight, drawn last so that the draws above do not depend on it
    norm_w = f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(L["head_dim"])).astype(np.float32))
    return dict(state=state, conv_cache=conv_cache, conv_w=conv_w, norm_w=norm_w, batch=batch, **L)


def decode_step_inputs(step, batch=256, seed=1003, conv_input=True, gate_input=False):
    """Inputs of decode step ``step`` (seeded by (seed, step)): q,k unit bf16, v bf16,
    g/beta fp32, (``conv_input``) the raw conv input x [batch, 10240] bf16 and
    (``gate_input``, drawn after x) the norm gate z [batch, 48, 128] bf16 ~ N(0, 1)."""
    L = LAYER
    rng = np.random.default_rng([seed, step])
    q = f32_to_bf16_bits(unit_vectors(rng, (batch, L["num_k_heads"], L["head_dim"])))
    k = f32_to_bf16_bits(unit_vectors(rng, (batch, L["num_k_heads"], L["head_dim"])))
    v = f32_to_bf16_bits(rng.standard_normal((batch, L["num_v_heads"], L["head_dim"]),
                                             dtype=np.float32))
    g, beta = gate_draws(rng, (batch, L["num_v_heads"]))
    out = dict(q=q, k=k, v=v, g=g, beta=beta)
    if conv_input:
        out["x"] = f32_to_bf16_bits(rng.standard_normal((batch, L["conv_channels"]), dtype=np.float32)
                                    * np.float32(PROJ_STD))
    if gate_input:
        out["z"] = f32_to_bf16_bits(rng.standard_normal((batch, L["num_v_heads"], L["head_dim"]),
                                                        dtype=np.float32))
    return out


def make_config(index, seed=None):
    """The five workloads of the layer (index 0..4), seeded with 1000 + index.

    0: fp32, one key group (1 key / 3 value heads), T = 512, zero initial state.
    1: full-layer prefill chain at T = 8192 (conv inputs, gates, norm gate/weight).
    2: long prefill, T = 65536, bf16, initial state N(0, 0.01^2).
    3: batched decode, 256 sequences: states, conv cache, conv weights
       (per-step inputs come from ``decode_step_inputs``).
    4: packed varlen prefill, 32 log-uniform lengths in [512, 32768], bf16,
       initial states zero for even and N(0, 0.01^2) for odd sequences.
    """
    rng = np.random.default_rng(1000 + index if seed is None else seed)
    L = LAYER
    if index == 0:
        return sequence_inputs(rng, [512], 1, 3, L["head_dim"], dtype="f32", init=None)
    if index == 1:
        return layer_prefill_inputs(rng, 8192)
    if index == 2:
        return sequence_inputs(rng, [65536], L["num_k_heads"], L["num_v_heads"], L["head_dim"],
                               dtype="bf16", init="normal")
    if index == 3:
        return decode_state_inputs(rng, 256)
    if index == 4:
        lengths = varlen_lengths(rng)
        return sequence_inputs(rng, lengths, L["num_k_heads"], L["num_v_heads"], L["head_dim"],
                               dtype="bf16", init="alternate")
    raise ValueError(f"no workload {index}")
