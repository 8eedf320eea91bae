"""gated_delta_rule_35_amd — the gated delta-rule layer on MI355X (gfx950).

Thin Python binding over the C ABI of libagnes_gdn (include/agnes_gdn.h).  The
functions below only check tensor layouts and pass device pointers, sizes and
the current HIP stream to the library; every step of the layer runs in the
library's HIP kernels.  torch supplies device memory and streams.

The layer (model card "Agnes-3.0-Flash Preview", 架构 table, delta-rule row;
discosf article "Agnes 3.0 Flash 刚上线就刷屏…", section 二.1):
  conv            kernel-4 causal depth-wise conv + SiLU (+ L2 norm of q/k heads)
  prefill_chunked chunked gated delta rule (chunk 64) over a packed batch
  prefill_fused   conv + SiLU + L2 and the chunked prefill in one call, from the raw q|k|v projection
  decode_step     stepwise gated delta rule, state updated in place
  gated_rmsnorm   y = rmsnorm(o) * w * silu(z)
  decode_fused    one decode token through conv, recurrence and norm in one call
The global attention layer of the same model (model card, rows 全局注意力 and 位置编码):
  attn_prefill    q/k RMS-norm + partial three-axis rotary, causal GQA softmax attention, sigmoid gate
  attn_decode     one token per entry against a bf16 KV cache (the new k, v written at index len)
"""
import ctypes

import torch

from . import _lib

__all__ = ["conv", "prefill_chunked", "prefill_fused", "decode_step", "gated_rmsnorm", "decode_fused",
           "prefill_workspace_size", "layer_prefill", "layer_prefill_workspace_size", "attn_prefill", "attn_prefill_workspace_size",
           "attn_decode", "attn_decode_workspace_size", "ceiling_rmw_stream", "ceiling_mfma", "workspace_status", "set_wait_limit", "set_prefill_stages",
           "WS_WAIT_LDS", "WS_WAIT_EXCHANGE", "WS_WAIT_ROLE", "WS_RANGE", "layer_prefill_noalloc",
           "AgnesError", "version", "LIB_PATH"]

LIB_PATH = _lib.LIB_PATH
HEAD_DIM = 128


class AgnesError(RuntimeError):
    def __init__(self, fn, status):
        lib = _lib.load()
        msg = lib.agnes_gdn_status_string(status).decode()
        if status == _lib.ERR_HIP:
            msg += f" (hipError_t {lib.agnes_gdn_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def _dt(t):
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check(fn, status):
    if status != _lib.OK:
        raise AgnesError(fn, status)


def _rows(t, name, width):
    """(token stride) of a [T, width] view whose last dim is contiguous."""
    if t.dim() != 2 or t.shape[1] != width or (t.numel() > 0 and t.shape[0] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name}: expected a [T, {width}] view with unit inner stride, got "
                         f"{tuple(t.shape)} / {t.stride()}")
    return t.stride(0) if t.numel() > 0 else width


def _heads(t, name, heads, dim=HEAD_DIM):
    """Token stride of a [T, heads, dim] view with contiguous heads."""
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != dim:
        raise ValueError(f"{name}: expected [T, {heads}, {dim}], got {tuple(t.shape)}")
    if t.numel() == 0:
        return heads * dim
    if t.stride(2) != 1 or (heads > 1 and t.stride(1) != dim):
        raise ValueError(f"{name}: heads must be contiguous (strides {t.stride()})")
    return t.stride(0) if t.shape[0] > 0 else heads * dim


def version():
    return _lib.load().agnes_gdn_version().decode()


def conv(x, weight, *, y=None, bias=None, cu_seqlens=None, conv_state=None, l2norm_heads=0,
         head_dim=HEAD_DIM, eps=1e-6):
    """Causal depth-wise conv (kernel 4) + SiLU (+ L2 norm of the leading ``l2norm_heads`` heads).

    x: [T, C] (row stride free, inner stride 1); weight: [C, 4] contiguous; bias: [C] or None.
    cu_seqlens: int32 [N+1] on the device (prefill), or None for decode mode (T sequences of
    one token, conv_state required).  conv_state: [N, C, 3] oldest first, updated in place.
    Returns y ([T, C], x's dtype, contiguous unless given).
    """
    T, C = x.shape
    xs = _rows(x, "x", C)
    if y is None:
        y = torch.empty((T, C), dtype=x.dtype, device=x.device)
    ys = _rows(y, "y", C)
    if weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight: expected a contiguous [C, K] tensor")
    for t, name in ((y, "y"), (weight, "weight"), (bias, "bias"), (conv_state, "conv_state")):
        if t is not None and t.dtype != x.dtype:
            raise TypeError(f"{name} must have x's dtype {x.dtype}")
    if conv_state is not None and not conv_state.is_contiguous():
        raise ValueError("conv_state must be contiguous [N, C, K-1]")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        n = cu_seqlens.numel() - 1
    else:
        n = T
    st = _lib.load().agnes_gdn_conv(
        _ptr(x), xs, _ptr(y), ys, _dt(x), _ptr(weight), _ptr(bias), _ptr(cu_seqlens), n, T, C,
        weight.shape[1], _ptr(conv_state), l2norm_heads, head_dim, eps, _stream(x.device))
    _check("agnes_gdn_conv", st)
    return y


def prefill_workspace_size(num_seqs, total_tokens, num_k_heads, num_v_heads, in_dtype):
    return _lib.load().agnes_gdn_prefill_workspace_size(
        num_seqs, total_tokens, num_k_heads, num_v_heads, HEAD_DIM,
        _lib.BF16 if in_dtype == torch.bfloat16 else _lib.F32)


def prefill_chunked(q, k, v, g, beta, cu_seqlens, *, initial_state=None, final_state=None,
                    output_final_state=True, scale=1.0, o=None, o_dtype=None, workspace=None):
    """Chunked gated delta-rule prefill over a packed batch.

    q, k: [T, Hk, 128]; v: [T, Hv, 128] (token strides free; views of a conv output work);
    g, beta: fp32 [T, Hv]; cu_seqlens: int32 [N+1] (device); initial_state: fp32
    [N, Hv, 128, 128] or None.  final_state: preallocated output (may be initial_state for
    an in-place update); allocated when None and ``output_final_state``.
    Returns (o [T, Hv, 128], final_state or None).
    """
    T, Hk, _ = q.shape
    Hv = v.shape[1]
    qs = _heads(q, "q", Hk)
    if _heads(k, "k", Hk) != qs:
        raise ValueError("q and k must share one token stride")
    vs = _heads(v, "v", Hv)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    for t, name in ((g, "g"), (beta, "beta")):
        if t.dtype != torch.float32 or tuple(t.shape) != (T, Hv) or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous fp32 [{T}, {Hv}]")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    n = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty((T, Hv, HEAD_DIM), dtype=o_dtype or q.dtype, device=q.device)
    elif not o.is_contiguous():
        raise ValueError("o must be contiguous")
    for s, name in ((initial_state, "initial_state"), (final_state, "final_state")):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous()
                              or tuple(s.shape) != (n, Hv, HEAD_DIM, HEAD_DIM)):
            raise ValueError(f"{name}: expected contiguous fp32 [{n}, {Hv}, 128, 128]")
    if final_state is None and output_final_state:
        final_state = torch.empty((n, Hv, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = prefill_workspace_size(n, T, Hk, Hv, q.dtype)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = _lib.load().agnes_gdn_prefill_chunked(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), qs, vs, _ptr(g), _ptr(beta), _ptr(cu_seqlens), n, T,
        Hk, Hv, HEAD_DIM, scale, _ptr(initial_state), _ptr(final_state), _ptr(o), _dt(o),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(q.device))
    _check("agnes_gdn_prefill_chunked", st)
    return o, final_state


def prefill_fused(x, conv_weight, g, beta, cu_seqlens, *, num_k_heads, conv_bias=None, conv_state=None,
                  initial_state=None, final_state=None, output_final_state=True, scale=1.0, l2norm_eps=1e-6,
                  o=None, o_dtype=None, workspace=None):
    """Causal conv (kernel 4) + SiLU + L2(q, k) and the chunked prefill in one call.

    x: bf16 [T, (2 Hk + Hv) * 128] raw projection output, channels q | k | v (row stride free,
    inner stride 1); conv_weight: [C, 4]; conv_bias: [C] or None; conv_state: [N, C, 3] (updated
    in place to each sequence's final history) or None; the rest as ``prefill_chunked``.
    Returns (o [T, Hv, 128], final_state or None).
    """
    T, C = x.shape
    Hk = num_k_heads
    Hv = C // HEAD_DIM - 2 * Hk
    if Hv <= 0 or C != (2 * Hk + Hv) * HEAD_DIM:
        raise ValueError(f"x: {C} channels do not hold 2 x {Hk} key heads and whole value heads")
    xs = _rows(x, "x", C)
    for t, name in ((conv_weight, "conv_weight"), (conv_bias, "conv_bias"), (conv_state, "conv_state")):
        if t is not None and (t.dtype != x.dtype or not t.is_contiguous()):
            raise ValueError(f"{name}: contiguous, with x's dtype {x.dtype}")
    if tuple(conv_weight.shape) != (C, 4):
        raise ValueError("conv_weight: [C, 4] expected")
    for t, name in ((g, "g"), (beta, "beta")):
        if t.dtype != torch.float32 or tuple(t.shape) != (T, Hv) or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous fp32 [{T}, {Hv}]")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    n = cu_seqlens.numel() - 1
    if conv_state is not None and tuple(conv_state.shape) != (n, C, 3):
        raise ValueError(f"conv_state: expected [{n}, {C}, 3]")
    if o is None:
        o = torch.empty((T, Hv, HEAD_DIM), dtype=o_dtype or x.dtype, device=x.device)
    elif not o.is_contiguous():
        raise ValueError("o must be contiguous")
    for s, name in ((initial_state, "initial_state"), (final_state, "final_state")):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous()
                              or tuple(s.shape) != (n, Hv, HEAD_DIM, HEAD_DIM)):
            raise ValueError(f"{name}: expected contiguous fp32 [{n}, {Hv}, 128, 128]")
    if final_state is None and output_final_state:
        final_state = torch.empty((n, Hv, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=x.device)
    need = prefill_workspace_size(n, T, Hk, Hv, torch.bfloat16)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    st = _lib.load().agnes_gdn_prefill_fused(
        _ptr(x), xs, _dt(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), _ptr(g), _ptr(beta),
        _ptr(cu_seqlens), n, T, Hk, Hv, HEAD_DIM, scale, l2norm_eps, _ptr(initial_state), _ptr(final_state),
        _ptr(o), _dt(o), _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(x.device))
    _check("agnes_gdn_prefill_fused", st)
    return o, final_state


def layer_prefill_workspace_size(num_seqs, total_tokens, num_k_heads, num_v_heads):
    return _lib.load().agnes_gdn_layer_prefill_workspace_size(num_seqs, total_tokens, num_k_heads, num_v_heads,
                                                              HEAD_DIM)


def layer_prefill(x, conv_weight, g, beta, cu_seqlens, z, norm_weight, *, num_k_heads, conv_bias=None,
                  conv_state=None, initial_state=None, final_state=None, output_final_state=True, scale=1.0,
                  l2norm_eps=1e-6, norm_eps=1e-6, y=None, o=None, out_dtype=None, workspace=None):
    """The whole delta-rule layer in prefill: conv + SiLU + L2(q, k), the chunked delta rule and
    the gated RMS-norm in one call (the recurrence output need not go to memory).

    x, conv_*, g, beta, cu_seqlens, states: as ``prefill_fused``; z: bf16 [T, Hv, 128] (heads
    contiguous, token stride free); norm_weight: bf16 [128].  o, if given, also receives the
    un-normalised recurrence output.  Returns (y [T, Hv, 128], final_state or None).
    """
    T, C = x.shape
    Hk = num_k_heads
    Hv = C // HEAD_DIM - 2 * Hk
    if Hv <= 0 or C != (2 * Hk + Hv) * HEAD_DIM:
        raise ValueError(f"x: {C} channels do not hold 2 x {Hk} key heads and whole value heads")
    xs = _rows(x, "x", C)
    zs = _heads(z, "z", Hv)
    for t, name in ((conv_weight, "conv_weight"), (conv_bias, "conv_bias"), (conv_state, "conv_state"),
                    (norm_weight, "norm_weight")):
        if t is not None and (t.dtype != x.dtype or not t.is_contiguous()):
            raise ValueError(f"{name}: contiguous, with x's dtype {x.dtype}")
    if tuple(conv_weight.shape) != (C, 4) or norm_weight.numel() != HEAD_DIM or z.dtype != x.dtype:
        raise ValueError("conv_weight [C, 4], norm_weight [128] and z of x's dtype expected")
    for t, name in ((g, "g"), (beta, "beta")):
        if t.dtype != torch.float32 or tuple(t.shape) != (T, Hv) or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous fp32 [{T}, {Hv}]")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    n = cu_seqlens.numel() - 1
    if conv_state is not None and tuple(conv_state.shape) != (n, C, 3):
        raise ValueError(f"conv_state: expected [{n}, {C}, 3]")
    out_dtype = out_dtype or (y.dtype if y is not None else x.dtype)
    if y is None:
        y = torch.empty((T, Hv, HEAD_DIM), dtype=out_dtype, device=x.device)
    for t, name in ((y, "y"), (o, "o")):
        if t is not None and (not t.is_contiguous() or t.dtype != out_dtype or tuple(t.shape) != (T, Hv, HEAD_DIM)):
            raise ValueError(f"{name}: contiguous {out_dtype} [{T}, {Hv}, 128] expected")
    for s, name in ((initial_state, "initial_state"), (final_state, "final_state")):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous()
                              or tuple(s.shape) != (n, Hv, HEAD_DIM, HEAD_DIM)):
            raise ValueError(f"{name}: expected contiguous fp32 [{n}, {Hv}, 128, 128]")
    if final_state is None and output_final_state:
        final_state = torch.empty((n, Hv, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=x.device)
    need = layer_prefill_workspace_size(n, T, Hk, Hv)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    st = _lib.load().agnes_gdn_layer_prefill(
        _ptr(x), xs, _dt(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), _ptr(g), _ptr(beta),
        _ptr(cu_seqlens), n, T, Hk, Hv, HEAD_DIM, scale, l2norm_eps, _ptr(initial_state), _ptr(final_state),
        _ptr(z), zs, _ptr(norm_weight), norm_eps, _ptr(y), _ptr(o), _dt(y), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(x.device))
    _check("agnes_gdn_layer_prefill", st)
    return y, final_state


def decode_step(q, k, v, g, beta, state, *, scale=1.0, o=None, o_dtype=None):
    """One stepwise decode token per sequence; ``state`` (fp32 [B, Hv, 128, 128]) is updated
    in place.  q, k: [B, Hk, 128]; v: [B, Hv, 128]; g, beta: fp32 [B, Hv].  Returns o."""
    B, Hk, _ = q.shape
    Hv = v.shape[1]
    qs = _heads(q, "q", Hk)
    if _heads(k, "k", Hk) != qs:
        raise ValueError("q and k must share one token stride")
    vs = _heads(v, "v", Hv)
    if state.dtype != torch.float32 or not state.is_contiguous() or tuple(state.shape) != (B, Hv, HEAD_DIM, HEAD_DIM):
        raise ValueError("state: expected contiguous fp32 [B, Hv, 128, 128]")
    for t, name in ((g, "g"), (beta, "beta")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, Hv) or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous fp32 [{B}, {Hv}]")
    if o is None:
        o = torch.empty((B, Hv, HEAD_DIM), dtype=o_dtype or q.dtype, device=q.device)
    st = _lib.load().agnes_gdn_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), qs, vs, _ptr(g), _ptr(beta), B, Hk, Hv, HEAD_DIM, scale,
        _ptr(state), _ptr(o), _dt(o), _stream(q.device))
    _check("agnes_gdn_decode_step", st)
    return o


def gated_rmsnorm(o, z, weight, *, eps=1e-6, y=None, y_dtype=None):
    """y = o / sqrt(mean(o^2) + eps) * weight * silu(z) per row of 128 (o, z contiguous)."""
    if o.shape[-1] != HEAD_DIM or z.shape != o.shape or not o.is_contiguous() or not z.is_contiguous():
        raise ValueError("o and z: contiguous tensors of one shape ending in 128")
    if weight.numel() != HEAD_DIM or weight.dtype != z.dtype:
        raise ValueError("weight: [128] with z's dtype")
    if y is None:
        y = torch.empty(o.shape, dtype=y_dtype or o.dtype, device=o.device)
    rows = o.numel() // HEAD_DIM
    st = _lib.load().agnes_gdn_gated_rmsnorm(
        _ptr(o), _dt(o), _ptr(z), _ptr(weight), _dt(z), eps, rows, HEAD_DIM, _ptr(y), _dt(y),
        _stream(o.device))
    _check("agnes_gdn_gated_rmsnorm", st)
    return y


def decode_fused(x, conv_weight, conv_state, g, beta, z, norm_weight, state, *, num_k_heads,
                 conv_bias=None, slots=None, scale=1.0, l2norm_eps=1e-6, norm_eps=1e-6, y=None,
                 o=None, y_dtype=None):
    """One decode token per batch entry through conv + SiLU + L2(q, k) + recurrence + gated norm.

    x: [B, (2 Hk + Hv) * 128] (row stride free, inner stride 1); conv_weight: [C, 4];
    conv_state: [S, C, 3] and state: fp32 [S, Hv, 128, 128] (both updated in place, S slots);
    g, beta: fp32 [B, Hv]; z: [B, Hv, 128]; norm_weight: [128]; slots: int32 [B] on the device
    or None (entry b uses slot b).  x, conv_weight, conv_bias, conv_state, z and norm_weight share
    one dtype.  o: optional [B, Hv, 128] output of the recurrence before the norm.  Returns y.
    """
    B, C = x.shape
    Hk = num_k_heads
    if state.dim() != 4 or state.shape[2:] != (HEAD_DIM, HEAD_DIM) or state.dtype != torch.float32 \
            or not state.is_contiguous():
        raise ValueError("state: expected contiguous fp32 [S, Hv, 128, 128]")
    S, Hv = state.shape[0], state.shape[1]
    if C != (2 * Hk + Hv) * HEAD_DIM:
        raise ValueError(f"x: expected {(2 * Hk + Hv) * HEAD_DIM} channels, got {C}")
    xs = _rows(x, "x", C)
    for t, name in ((conv_weight, "conv_weight"), (conv_bias, "conv_bias"), (conv_state, "conv_state"),
                    (z, "z"), (norm_weight, "norm_weight")):
        if t is not None and (t.dtype != x.dtype or not t.is_contiguous()):
            raise ValueError(f"{name}: contiguous, with x's dtype {x.dtype}")
    if tuple(conv_weight.shape) != (C, 4) or tuple(conv_state.shape) != (S, C, 3):
        raise ValueError("conv_weight [C, 4] and conv_state [S, C, 3] expected")
    if tuple(z.shape) != (B, Hv, HEAD_DIM) or norm_weight.numel() != HEAD_DIM:
        raise ValueError("z [B, Hv, 128] and norm_weight [128] expected")
    for t, name in ((g, "g"), (beta, "beta")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, Hv) or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous fp32 [{B}, {Hv}]")
    if slots is not None and (slots.dtype != torch.int32 or slots.numel() != B or not slots.is_contiguous()):
        raise ValueError("slots: contiguous int32 [B]")
    if y is None:
        y = torch.empty((B, Hv, HEAD_DIM), dtype=y_dtype or x.dtype, device=x.device)
    for t, name in ((y, "y"), (o, "o")):
        if t is not None and (tuple(t.shape) != (B, Hv, HEAD_DIM) or not t.is_contiguous() or t.dtype != y.dtype):
            raise ValueError(f"{name}: contiguous [B, Hv, 128] of one dtype")
    st = _lib.load().agnes_gdn_decode_fused(
        _ptr(x), xs, _dt(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), _ptr(g), _ptr(beta),
        _ptr(z), _ptr(norm_weight), _ptr(state), _ptr(slots), S, B, Hk, Hv, HEAD_DIM, scale, l2norm_eps,
        norm_eps, _ptr(y), _ptr(o), _dt(y), _stream(x.device))
    _check("agnes_gdn_decode_fused", st)
    return y


ATTN_HEAD_DIM = 256
ATTN_ROT_DIM = 64


def attn_prefill_workspace_size(num_seqs, total_tokens):
    return int(_lib.load().agnes_attn_prefill_workspace_size(num_seqs, total_tokens))


def attn_prefill(q, k, v, gate, q_norm_weight, k_norm_weight, cu_seqlens, *, positions=None, k_out=None,
                 v_out=None, rope_base=1e7, norm_eps=1e-6, scale=0.0, o=None, o_dtype=None, workspace=None):
    """Global attention layer over a packed batch (prefill).

    q, gate: bf16 [T, Hq, 256]; k, v: bf16 [T, Hkv, 256] (token strides free, heads contiguous);
    norm weights: bf16 [256]; cu_seqlens: int32 [N+1] (device); positions: int32 [3, T] or None
    (text positions).  k_out: bf16 [T, Hkv, 256] view receiving the normalised, rotated k (the KV
    cache rows; allocated when None); v_out: optional copy of v.  scale <= 0 selects 1/16.
    Returns (o [T, Hq, 256], k_out).
    """
    T, Hq, _ = q.shape
    Hkv = k.shape[1]
    strides = {}
    for t, name, h in ((q, "q", Hq), (gate, "gate", Hq), (k, "k", Hkv), (v, "v", Hkv)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
        strides[name] = _heads(t, name, h, ATTN_HEAD_DIM)
    for t, name in ((q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight")):
        if t.dtype != torch.bfloat16 or t.numel() != ATTN_HEAD_DIM or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous bf16 [256]")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    n = cu_seqlens.numel() - 1
    ps = 0
    if positions is not None:
        if positions.dtype != torch.int32 or positions.dim() != 2 or positions.shape[0] != 3 \
                or positions.shape[1] != T or positions.stride(1) != 1:
            raise ValueError("positions: expected int32 [3, T] with unit inner stride")
        ps = positions.stride(0)
    if k_out is None:
        k_out = torch.empty((T, Hkv, ATTN_HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    kos = _heads(k_out, "k_out", Hkv, ATTN_HEAD_DIM)
    vos = 0 if v_out is None else _heads(v_out, "v_out", Hkv, ATTN_HEAD_DIM)
    if o is None:
        o = torch.empty((T, Hq, ATTN_HEAD_DIM), dtype=o_dtype or torch.bfloat16, device=q.device)
    elif not o.is_contiguous():
        raise ValueError("o must be contiguous")
    need = attn_prefill_workspace_size(n, T)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = _lib.load().agnes_attn_prefill(
        _ptr(q), strides["q"], _ptr(k), strides["k"], _ptr(v), strides["v"], _ptr(gate), strides["gate"],
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions), ps, _ptr(cu_seqlens), n, T, Hq, Hkv,
        ATTN_HEAD_DIM, ATTN_ROT_DIM, rope_base, norm_eps, scale, _ptr(k_out), kos, _ptr(v_out), vos,
        _ptr(o), _dt(o), _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(q.device))
    _check("agnes_attn_prefill", st)
    return o, k_out


def attn_decode_workspace_size(batch, num_q_heads, num_kv_heads, max_len):
    return int(_lib.load().agnes_attn_decode_workspace_size(batch, num_q_heads, num_kv_heads, max_len))


def attn_decode(q, k, v, gate, q_norm_weight, k_norm_weight, k_cache, v_cache, cache_lens, *, positions=None,
                rope_base=1e7, norm_eps=1e-6, scale=0.0, o=None, o_dtype=None, workspace=None):
    """One decode step of the global attention layer.

    q, gate: bf16 [B, Hq, 256]; k, v: bf16 [B, Hkv, 256]; caches: contiguous bf16
    [B, max_len, Hkv, 256] (row cache_lens[b] of entry b is written); cache_lens: int32 [B]
    (device; entries outside [0, max_len) are padding); positions: int32 [3, B] or None.
    Returns o [B, Hq, 256].  The caller advances cache_lens.
    """
    B, Hq, _ = q.shape
    Hkv = k.shape[1]
    strides = {}
    for t, name, h in ((q, "q", Hq), (gate, "gate", Hq), (k, "k", Hkv), (v, "v", Hkv)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
        strides[name] = _heads(t, name, h, ATTN_HEAD_DIM)
    for c, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if c.dtype != torch.bfloat16 or c.dim() != 4 or tuple(c.shape[::2]) != (B, Hkv) \
                or c.shape[3] != ATTN_HEAD_DIM or not c.is_contiguous():
            raise ValueError(f"{name}: expected contiguous bf16 [{B}, max_len, {Hkv}, 256]")
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    max_len = k_cache.shape[1]
    if cache_lens.dtype != torch.int32 or cache_lens.numel() != B:
        raise ValueError(f"cache_lens: expected int32 [{B}]")
    for t, name in ((q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight")):
        if t.dtype != torch.bfloat16 or t.numel() != ATTN_HEAD_DIM or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous bf16 [256]")
    ps = 0
    if positions is not None:
        if positions.dtype != torch.int32 or positions.dim() != 2 or positions.shape[0] != 3 \
                or positions.shape[1] != B or positions.stride(1) != 1:
            raise ValueError("positions: expected int32 [3, B] with unit inner stride")
        ps = positions.stride(0)
    if o is None:
        o = torch.empty((B, Hq, ATTN_HEAD_DIM), dtype=o_dtype or torch.bfloat16, device=q.device)
    elif not o.is_contiguous():
        raise ValueError("o must be contiguous")
    need = attn_decode_workspace_size(B, Hq, Hkv, max_len)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = _lib.load().agnes_attn_decode(
        _ptr(q), strides["q"], _ptr(k), strides["k"], _ptr(v), strides["v"], _ptr(gate), strides["gate"],
        _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions), ps, _ptr(k_cache), _ptr(v_cache), max_len,
        _ptr(cache_lens), B, Hq, Hkv, ATTN_HEAD_DIM, ATTN_ROT_DIM, rope_base, norm_eps, scale, _ptr(o), _dt(o),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(q.device))
    _check("agnes_attn_decode", st)
    return o


def ceiling_rmw_stream(buf):
    """Measurement kernel: every 16-byte vector of the device tensor ``buf`` read and written back
    once (contents unchanged); 2 * buf's bytes move through HBM."""
    nbytes = buf.numel() * buf.element_size()
    _check("agnes_gdn_ceiling_rmw_stream",
           _lib.load().agnes_gdn_ceiling_rmw_stream(buf.data_ptr(), nbytes, _stream(buf.device)))


def ceiling_mfma(sink, blocks, iters):
    """Measurement kernel: ``blocks`` workgroups of four waves, each issuing ``iters`` rounds of 8
    independent bf16 16x16x32 matrix-core products held in registers
    (blocks * 4 * iters * 8 * 16384 FLOPs); ``sink`` is a float32 device tensor of blocks * 4."""
    if sink.dtype != torch.float32 or sink.numel() < 4 * blocks:
        raise ValueError("sink: float32 tensor of at least 4 * blocks elements")
    _check("agnes_gdn_ceiling_mfma",
           _lib.load().agnes_gdn_ceiling_mfma(sink.data_ptr(), blocks, iters, _stream(sink.device)))


WS_WAIT_LDS, WS_WAIT_EXCHANGE, WS_WAIT_ROLE, WS_RANGE = (_lib.WS_WAIT_LDS, _lib.WS_WAIT_EXCHANGE, _lib.WS_WAIT_ROLE,
                                                         _lib.WS_RANGE)


def workspace_status(workspace):
    """Status bits (WS_WAIT_LDS, WS_WAIT_EXCHANGE, WS_WAIT_ROLE, WS_RANGE) that the last bf16 prefill
    call on ``workspace`` (a device uint8 tensor passed as its workspace) left in it; 0 when all is
    well.  Synchronises the current stream."""
    flags = ctypes.c_uint32(0)
    _check("agnes_gdn_workspace_status",
           _lib.load().agnes_gdn_workspace_status(workspace.data_ptr(), ctypes.addressof(flags),
                                                  _stream(workspace.device)))
    return flags.value


def set_wait_limit(polls):
    """Process-wide bound on the polls of the bf16 prefill calls' bounded waits (0 restores each
    wait's own bound).  For tests of the status bits only: with a small bound the waits give up
    and the results are unreliable."""
    _check("agnes_gdn_set_wait_limit", _lib.load().agnes_gdn_set_wait_limit(int(polls)))



def set_prefill_stages(cuts=None):
    """Process-wide stage cuts of the bf16 prefill calls, in 1/40ths of each sequence's chunks
    (strictly increasing inside (0, 40), at most 7; () runs every call in one stage), for every
    kind of call.  None restores the defaults: two stages, cut at 26 for the whole-layer calls
    and at 28 for the prefill calls.  The cuts change the schedule only, not the results."""
    if cuts is None:
        _check("agnes_gdn_set_prefill_stages", _lib.load().agnes_gdn_set_prefill_stages(None, -1))
        return
    arr = (ctypes.c_int32 * max(len(cuts), 1))(*[int(c) for c in cuts])
    _check("agnes_gdn_set_prefill_stages", _lib.load().agnes_gdn_set_prefill_stages(arr, len(cuts)))

def layer_prefill_noalloc(x, conv_weight, g, beta, cu_seqlens, z, norm_weight, y, *, num_k_heads, conv_bias=None,
                          conv_state=None, initial_state=None, final_state=None, scale=1.0, l2norm_eps=1e-6,
                          norm_eps=1e-6, o=None):
    """``layer_prefill`` for callers that cannot allocate: the library's fixed per-device workspace
    (64 MiB: one sequence of up to about 2400 tokens) replaces the workspace argument, and nothing is
    allocated, here or in the library.  Every output (y, and final_state / o if wanted) is given by
    the caller.  Calls that overlap in time on one device race.  Returns y."""
    T, C = x.shape
    Hk = num_k_heads
    Hv = C // HEAD_DIM - 2 * Hk
    if Hv <= 0 or C != (2 * Hk + Hv) * HEAD_DIM:
        raise ValueError(f"x: {C} channels do not hold 2 x {Hk} key heads and whole value heads")
    if y is None or tuple(y.shape) != (T, Hv, HEAD_DIM) or not y.is_contiguous():
        raise ValueError(f"y: contiguous [{T}, {Hv}, 128] expected")
    for t, name in ((o, "o"),):
        if t is not None and (not t.is_contiguous() or t.dtype != y.dtype or tuple(t.shape) != (T, Hv, HEAD_DIM)):
            raise ValueError(f"{name}: contiguous {y.dtype} [{T}, {Hv}, 128] expected")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    n = cu_seqlens.numel() - 1
    for s, name in ((initial_state, "initial_state"), (final_state, "final_state")):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous()
                              or tuple(s.shape) != (n, Hv, HEAD_DIM, HEAD_DIM)):
            raise ValueError(f"{name}: expected contiguous fp32 [{n}, {Hv}, 128, 128]")
    st = _lib.load().agnes_gdn_layer_prefill_noalloc(
        _ptr(x), _rows(x, "x", C), _dt(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), _ptr(g), _ptr(beta),
        _ptr(cu_seqlens), n, T, Hk, Hv, HEAD_DIM, scale, l2norm_eps, _ptr(initial_state), _ptr(final_state),
        _ptr(z), _heads(z, "z", Hv), _ptr(norm_weight), norm_eps, _ptr(y), _ptr(o), _dt(y), _stream(x.device))
    _check("agnes_gdn_layer_prefill_noalloc", st)
    return y
