"""GPU checks of the status word of the bf16 prefill calls (agnes_gdn_workspace_status).

A correct call leaves it clear.  A process-wide poll bound of 1 (agnes_gdn_set_wait_limit) makes
the bounded waits give up from the host's side: the kernels still end normally, the word reports
it, and a later call with the default bound is clear and correct again.  Values outside the fp16
range of the matrix-core path set the range bit.  No test here faults, traps or hangs the GPU:
every wait is bounded and every out-of-range value is an ordinary floating-point number.
"""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits
from synth.configs import sequence_inputs
from tests.helpers import dev, host, rel_l2

torch = pytest.importorskip("torch")
import gated_delta_rule_35_amd as gdn  # noqa: E402

pytestmark = pytest.mark.gpu

D = 128


def _layer_case(rng, lens, hk, hv, scale=1.43):
    T = int(sum(lens))
    C = (2 * hk + hv) * D
    f = np.float32
    return dict(
        x=f32_to_bf16_bits(rng.standard_normal((T, C)).astype(f) * f(scale)),
        w=f32_to_bf16_bits(rng.uniform(-0.5, 0.5, (C, 4)).astype(f)),
        g=(-0.05 * np.logaddexp(0, rng.standard_normal((T, hv)))).astype(f),
        beta=(1 / (1 + np.exp(-rng.standard_normal((T, hv))))).astype(f),
        z=f32_to_bf16_bits(rng.standard_normal((T, hv, D)).astype(f)),
        nw=f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(D)).astype(f)),
        cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), hk=hk, hv=hv)


def _layer(d, ws):
    y, fin = gdn.layer_prefill(dev(d["x"]), dev(d["w"]), dev(d["g"]), dev(d["beta"]), dev(d["cu"]), dev(d["z"]),
                               dev(d["nw"]), num_k_heads=d["hk"], out_dtype=torch.float32, workspace=ws)
    return y, fin


def _ws(d):
    T = d["g"].shape[0]
    return torch.empty(gdn.layer_prefill_workspace_size(len(d["cu"]) - 1, T, d["hk"], d["hv"]), dtype=torch.uint8,
                       device="cuda")


@pytest.fixture
def default_limit():
    yield
    gdn.set_wait_limit(0)


def test_status_clear_after_correct_calls():
    rng = np.random.default_rng(900)
    d = _layer_case(rng, [300, 70], 2, 6)
    ws = _ws(d)
    _layer(d, ws)
    assert gdn.workspace_status(ws) == 0
    s = sequence_inputs(rng, [200, 1, 90], 2, 6, D, dtype="bf16", init="normal")
    wsp = torch.empty(gdn.prefill_workspace_size(3, 291, 2, 6, torch.bfloat16), dtype=torch.uint8, device="cuda")
    gdn.prefill_chunked(dev(s["q"]), dev(s["k"]), dev(s["v"]), dev(s["g"]), dev(s["beta"]), dev(s["cu_seqlens"]),
                        initial_state=dev(s["initial_state"]), workspace=wsp)
    assert gdn.workspace_status(wsp) == 0


def test_waits_that_give_up_are_reported_and_kernels_end(default_limit):
    """Poll bound 1: the whole-layer call's waits give up (its y is then unreliable and not
    checked), every kernel ends, the word has wait bits; with the default bound again the same
    workspace gives a clear word and the oracle's result."""
    rng = np.random.default_rng(901)
    d = _layer_case(rng, [700, 130, 64], 2, 6)
    ws = _ws(d)
    gdn.set_wait_limit(1)
    _layer(d, ws)
    torch.cuda.synchronize()
    flags = gdn.workspace_status(ws)
    print(f"status with a poll bound of 1: {flags:#x}")
    assert flags & (gdn.WS_WAIT_LDS | gdn.WS_WAIT_EXCHANGE | gdn.WS_WAIT_ROLE)
    assert not flags & gdn.WS_RANGE
    gdn.set_wait_limit(0)
    y, fin = _layer(d, ws)
    assert gdn.workspace_status(ws) == 0
    ro, _, rf = oracle.prefill_conv_recurrence(d["x"], d["w"], d["cu"], None, d["g"], d["beta"], None, d["hk"], d["hv"])
    ry = oracle.gated_rmsnorm(ro, d["z"], d["nw"])
    assert rel_l2(host(y), ry) <= 2e-3 and rel_l2(host(fin), rf) <= 2e-3


def test_timing_hint_wait_giving_up_leaves_the_plain_prefill_exact(default_limit):
    """In the plain prefill the only bounded wait orders work in time (every hand-over of data goes
    through a workgroup barrier): when it gives up the word says so and the outputs are unchanged,
    bit for bit."""
    rng = np.random.default_rng(902)
    s = sequence_inputs(rng, [300, 65], 2, 6, D, dtype="bf16", init="normal")
    args = [dev(s[k]) for k in ("q", "k", "v", "g", "beta", "cu_seqlens")]
    ws = torch.empty(gdn.prefill_workspace_size(2, 365, 2, 6, torch.bfloat16), dtype=torch.uint8, device="cuda")
    o1, f1 = gdn.prefill_chunked(*args, initial_state=dev(s["initial_state"]), o_dtype=torch.float32, workspace=ws)
    o1, f1 = host(o1), host(f1)
    assert gdn.workspace_status(ws) == 0
    gdn.set_wait_limit(1)
    o2, f2 = gdn.prefill_chunked(*args, initial_state=dev(s["initial_state"]), o_dtype=torch.float32, workspace=ws)
    flags = gdn.workspace_status(ws)
    gdn.set_wait_limit(0)
    np.testing.assert_array_equal(host(o2), o1)
    np.testing.assert_array_equal(host(f2), f1)
    assert flags & gdn.WS_WAIT_LDS and not flags & gdn.WS_RANGE


@pytest.mark.parametrize("what", ["q_magnitude", "positive_decay", "state_magnitude"])
def test_fp16_range_is_reported(what):
    """q of magnitude 2^17 (plain call); log-decays of +1 per token (the in-chunk decay factors reach
    e^63); an initial state of magnitude 10^5.  Each sets the range bit."""
    rng = np.random.default_rng(903)
    s = sequence_inputs(rng, [130], 1, 3, D, dtype="bf16", init="normal")
    q, g, s0 = s["q"].copy(), s["g"].copy(), s["initial_state"].copy()
    if what == "q_magnitude":
        q[5, 0, 7] = f32_to_bf16_bits(np.array([131072.0], np.float32))[0]
    elif what == "positive_decay":
        g[:] = 1.0
    else:
        s0[0, 1, 3, 4] = 1e5
    ws = torch.empty(gdn.prefill_workspace_size(1, 130, 1, 3, torch.bfloat16), dtype=torch.uint8, device="cuda")
    gdn.prefill_chunked(dev(q), dev(s["k"]), dev(s["v"]), dev(g), dev(s["beta"]), dev(s["cu_seqlens"]),
                        initial_state=dev(s0), workspace=ws)
    flags = gdn.workspace_status(ws)
    print(f"{what}: status {flags:#x}")
    assert flags & gdn.WS_RANGE


def test_release_then_calls_in_two_stages_again():
    """agnes_gdn_release destroys the side stream and events of the calls in two stages; the next
    such call creates them again and gives the same result bit for bit."""
    rng = np.random.default_rng(904)
    d = _layer_case(rng, [2000, 700], 2, 6)
    ws = _ws(d)
    y1, f1 = _layer(d, ws)
    y1, f1 = host(y1), host(f1)
    assert gdn._lib.load().agnes_gdn_release() == 0
    assert gdn._lib.load().agnes_gdn_release() == 0  # nothing left: no HIP call
    y2, f2 = _layer(d, ws)
    np.testing.assert_array_equal(host(y2), y1)
    np.testing.assert_array_equal(host(f2), f1)
    assert gdn.workspace_status(ws) == 0
