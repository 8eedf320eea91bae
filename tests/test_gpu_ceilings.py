"""GPU checks of the two measurement kernels the benchmark's ceilings come from.

The read + write stream must leave its buffer unchanged bit for bit (it multiplies by 1.0) over a
size that is not a multiple of its grid; the matrix-core loop gives every workgroup the same
operands, so every wave of one position in the workgroup must store the same finite value.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
import gated_delta_rule_35_amd as gdn  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n4", [1, 1000, 262144 + 7])
def test_rmw_stream_leaves_the_buffer_unchanged(n4):
    g = torch.Generator(device="cuda").manual_seed(n4)
    buf = torch.randn(4 * n4, device="cuda", generator=g)
    buf[::97] = float("-inf")
    buf[1::89] = -0.0
    ref = buf.clone()
    gdn.ceiling_rmw_stream(buf)
    torch.cuda.synchronize()
    assert torch.equal(buf.view(torch.int32), ref.view(torch.int32))


def test_mfma_loop_stores_one_finite_value_per_wave_position():
    blocks, iters = 37, 64
    sink = torch.full((4 * blocks,), float("nan"), device="cuda")
    gdn.ceiling_mfma(sink, blocks, iters)
    torch.cuda.synchronize()
    s = sink.cpu().numpy().reshape(blocks, 4)
    assert np.isfinite(s).all() and (s != 0).any()
    assert (s == s[0]).all()
