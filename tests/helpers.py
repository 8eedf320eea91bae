"""Shared test helpers: device transfer of generator bytes and comparison metrics."""
import numpy as np

from synth import f32_to_bf16_bits


def dev(a, device="cuda"):
    """numpy array -> device tensor with the same bytes (uint16 arrays become bfloat16)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t):
    """device tensor -> numpy (bfloat16 tensors come back as uint16 bit patterns)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_l2(x, ref):
    """||x - ref|| / ||ref|| (absolute max error when ref is all zero)."""
    x, ref = as_f64(x), as_f64(ref)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / n) if n > 0 else float(np.abs(x - ref).max())


def _ordered(bits):
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_ulps(gpu_bits, ref):
    """Distance in bf16 ulps between GPU bf16 results and the round-to-nearest-even of ref."""
    rb = f32_to_bf16_bits(np.asarray(ref, np.float64).astype(np.float32))
    return np.abs(_ordered(np.asarray(gpu_bits, np.uint16)) - _ordered(rb))
