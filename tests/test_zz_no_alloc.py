"""GPU check of agnes_gdn_layer_prefill_noalloc (the whole-layer prefill on the library's fixed
per-device workspace) against agnes_gdn_layer_prefill on its own workspace: two calls in a row,
the second on a smaller problem, each equal to the workspace call bit for bit (both compute the
same arithmetic; the fixed-workspace call always runs in one stage, which gives the two-stage
result bit for bit).  A problem whose workspace exceeds the fixed one is refused before anything
is launched."""
import numpy as np
import pytest

from synth import f32_to_bf16_bits
from tests.helpers import dev, host

torch = pytest.importorskip("torch")
import gated_delta_rule_35_amd as gdn  # noqa: E402
from gated_delta_rule_35_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu

D = 128


def _case(rng, lens, hk, hv):
    T = int(sum(lens))
    C = (2 * hk + hv) * D
    f = np.float32
    return dict(
        x=f32_to_bf16_bits(rng.standard_normal((T, C)).astype(f) * f(1.43)),
        w=f32_to_bf16_bits(rng.uniform(-0.5, 0.5, (C, 4)).astype(f)),
        cs=f32_to_bf16_bits(rng.standard_normal((len(lens), C, 3)).astype(f) * f(1.43)),
        g=(-0.05 * np.logaddexp(0, rng.standard_normal((T, hv)))).astype(f),
        beta=(1 / (1 + np.exp(-rng.standard_normal((T, hv))))).astype(f),
        s0=(rng.standard_normal((len(lens), hv, D, D)) * 0.01).astype(f),
        z=f32_to_bf16_bits(rng.standard_normal((T, hv, D)).astype(f)),
        nw=f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(D)).astype(f)),
        cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), hk=hk, hv=hv)


def _both(d):
    T, hv = d["g"].shape
    n = len(d["cu"]) - 1
    x, w, g, be, cu, z, nw, s0 = (dev(d[k]) for k in ("x", "w", "g", "beta", "cu", "z", "nw", "s0"))
    cs1, cs2 = dev(d["cs"]), dev(d["cs"])
    y1, f1 = gdn.layer_prefill(x, w, g, be, cu, z, nw, num_k_heads=d["hk"], conv_state=cs1, initial_state=s0,
                               out_dtype=torch.float32)
    y2 = torch.full((T, hv, D), float("nan"), dtype=torch.float32, device="cuda")
    f2 = torch.full((n, hv, D, D), float("nan"), dtype=torch.float32, device="cuda")
    gdn.layer_prefill_noalloc(x, w, g, be, cu, z, nw, y2, num_k_heads=d["hk"], conv_state=cs2, initial_state=s0,
                              final_state=f2)
    torch.cuda.synchronize()
    return (host(y1), host(f1), host(cs1)), (host(y2), host(f2), host(cs2))


def test_noalloc_equals_workspace_call_twice_second_smaller():
    rng = np.random.default_rng(950)
    big = _case(rng, [2000], 16, 48)          # the layer's heads, one 2000-token sequence (53 MB workspace)
    small = _case(rng, [300, 77, 1], 2, 6)    # then a smaller, ragged batch on the same fixed workspace
    need = gdn.layer_prefill_workspace_size(1, 2000, 16, 48)
    assert 0 < need <= 64 << 20
    for d in (big, small):
        (y1, f1, c1), (y2, f2, c2) = _both(d)
        np.testing.assert_array_equal(y2, y1)
        np.testing.assert_array_equal(f2, f1)
        np.testing.assert_array_equal(c2, c1)


def test_noalloc_refuses_problems_beyond_its_workspace():
    T = 8192
    assert gdn.layer_prefill_workspace_size(1, T, 16, 48) > 64 << 20
    x = torch.zeros((T, 80 * D), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((T, 48, D), dtype=torch.float32, device="cuda")
    st = _lib.load().agnes_gdn_layer_prefill_noalloc(
        x.data_ptr(), 80 * D, _lib.BF16, x.data_ptr(), None, None, y.data_ptr(), y.data_ptr(),
        torch.tensor([0, T], dtype=torch.int32, device="cuda").data_ptr(), 1, T, 16, 48, D, 1.0, 1e-6, None, None,
        x.data_ptr(), 48 * D, x.data_ptr(), 1e-6, y.data_ptr(), None, _lib.F32, None)
    assert st == _lib.ERR_UNSUPPORTED
