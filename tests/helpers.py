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


def check_bf16_out(gpu_bits, ref, abs_tol=0.0, exact_frac=0.999):
    """bf16 results against the fp64 reference: bit-exact (equal to RNE(ref)) for at least
    ``exact_frac`` of the elements, and each element within one bf16 ulp of RNE(ref) or within
    ``abs_tol`` of ref.  ``abs_tol`` covers results that fp32 arithmetic cannot round correctly
    (cancellation in a short fp32 sum leaves an absolute, not a relative, error)."""
    ref = np.asarray(ref, np.float64)
    u = bf16_ulps(gpu_bits, ref)
    exact = float((u == 0).mean())
    bad = u > 1
    if bad.any():
        err = np.abs(as_f64(np.asarray(gpu_bits)[bad]) - ref[bad])
        assert err.max() <= abs_tol, f"{int(bad.sum())} elements > 1 ulp, max abs err {err.max():.3e}"
    assert exact >= exact_frac, f"bit-exact fraction {exact}"
    return exact
