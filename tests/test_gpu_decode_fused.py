"""GPU parity of agnes_gdn_decode_fused (conv + SiLU + L2(q, k) + recurrence + gated norm in one
call) against the fp64 layer oracle on identical input bytes.

Tolerances: every step runs in fp32 with nothing rounded in between, so the fp32 `y`, `o` and
states are gated at rel-L2 1e-5 (as the unfused decode step); the bf16 `y` of the same call must
be the round-to-nearest-even of the fp32 `y` bit for bit; the conv history is a copy of input
values and must match exactly.
"""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits, make_config, decode_step_inputs
from tests.helpers import dev, host, rel_l2

torch = pytest.importorskip("torch")
import gated_delta_rule_35_amd as gdn  # noqa: E402

pytestmark = pytest.mark.gpu

D = 128


def _case(rng, B, hk, hv, S, dtype, bias=False):
    C = (2 * hk + hv) * D
    conv = f32_to_bf16_bits if dtype == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))
    f = np.float32
    d = dict(
        x=conv(rng.standard_normal((B, C)).astype(f) * f(1.43)),
        w=conv(rng.uniform(-0.5, 0.5, (C, 4)).astype(f)),
        b=conv(rng.uniform(-0.2, 0.2, C).astype(f)) if bias else None,
        cs=conv(rng.standard_normal((S, C, 3)).astype(f) * f(1.43)),
        g=(-0.05 * np.logaddexp(0, rng.standard_normal((B, hv)))).astype(f),
        beta=(1 / (1 + np.exp(-rng.standard_normal((B, hv))))).astype(f),
        z=conv(rng.standard_normal((B, hv, D)).astype(f)),
        nw=conv((1 + 0.1 * rng.standard_normal(D)).astype(f)),
        st=(rng.standard_normal((S, hv, D, D)) * 0.03).astype(f),
    )
    return d


def _run(d, hk, slots, y_dtype, cs, st, want_o=True, scale=1.0):
    B = d["x"].shape[0]
    hv = d["st"].shape[1]
    o = torch.empty((B, hv, D), dtype=y_dtype, device="cuda") if want_o else None
    y = gdn.decode_fused(dev(d["x"]), dev(d["w"]), cs, dev(d["g"]), dev(d["beta"]), dev(d["z"]), dev(d["nw"]), st,
                         num_k_heads=hk, conv_bias=None if d["b"] is None else dev(d["b"]),
                         slots=None if slots is None else dev(np.asarray(slots, np.int32)), y_dtype=y_dtype, o=o,
                         scale=scale)
    torch.cuda.synchronize()
    return host(y), (host(o) if want_o else None)


def _oracle(d, hk, slots, cs, st, scale=1.0):
    hv = d["st"].shape[1]
    return oracle.decode_layer_step(d["x"], d["w"], cs, d["g"], d["beta"], d["z"], d["nw"], st, hk, hv,
                                    slots=slots, conv_bias=d["b"], scale=scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_fused_steps_with_slots_and_padding(dtype):
    """Three consecutive steps on a pool of 9 slots: permuted slots, one entry past the pool
    and one negative (padding); caches carried on the GPU and in the oracle independently."""
    rng = np.random.default_rng(300)
    B, hk, hv, S = 6, 2, 6, 9
    d = _case(rng, B, hk, hv, S, dtype)
    slots = [7, 2, -1, 0, 11, 4]
    cs, st = dev(d["cs"]), dev(d["st"])
    rcs, rst = oracle.as_f64(d["cs"]), d["st"].astype(np.float64)
    for step in range(3):
        if step:
            d.update({k: v for k, v in _case(np.random.default_rng(300 + step), B, hk, hv, S, dtype).items()
                      if k in ("x", "g", "beta", "z")})
        y, o = _run(d, hk, slots, torch.float32, cs, st, scale=0.8)
        ry, ro, rcs, rst = _oracle(d, hk, slots, rcs, rst, scale=0.8)
        assert rel_l2(y, ry) <= 1e-5, step
        assert rel_l2(o, ro) <= 1e-5, step
        assert not y[[2, 4]].any() and not o[[2, 4]].any()
        np.testing.assert_array_equal(oracle.as_f64(host(cs)), rcs)
        assert rel_l2(host(st), rst) <= 1e-5
        np.testing.assert_array_equal(host(st)[[1, 3, 5, 6, 8]], d["st"][[1, 3, 5, 6, 8]])


@pytest.mark.parametrize("hk,hv,bias", [(1, 1, False), (2, 4, True), (1, 5, False), (3, 3, True), (1, 7, False),
                                        (1, 130, True)])
def test_decode_fused_group_sizes(hk, hv, bias):
    """Value heads per key head 1, 2, 5, 7 and 130 (each of them convolving the key head's q and
    k from the old history, which the second launch then advances), with and without conv bias;
    slots = None (entry b uses slot b)."""
    rng = np.random.default_rng(310 + 10 * hk + hv)
    B = 4
    d = _case(rng, B, hk, hv, B, "bf16", bias)
    cs, st = dev(d["cs"]), dev(d["st"])
    y, o = _run(d, hk, None, torch.float32, cs, st)
    ry, ro, rcs, rst = _oracle(d, hk, None, d["cs"], d["st"])
    assert rel_l2(y, ry) <= 1e-5 and rel_l2(o, ro) <= 1e-5
    assert rel_l2(host(st), rst) <= 1e-5
    np.testing.assert_array_equal(oracle.as_f64(host(cs)), rcs)


def test_decode_fused_bf16_output_is_rne_of_fp32_output():
    rng = np.random.default_rng(320)
    B, hk, hv, S = 5, 2, 6, 5
    d = _case(rng, B, hk, hv, S, "bf16")
    y32, o32 = _run(d, hk, None, torch.float32, dev(d["cs"]), dev(d["st"]))
    y16, o16 = _run(d, hk, None, torch.bfloat16, dev(d["cs"]), dev(d["st"]))
    np.testing.assert_array_equal(y16, f32_to_bf16_bits(y32))
    np.testing.assert_array_equal(o16, f32_to_bf16_bits(o32))


def test_decode_fused_equals_unfused_chain_in_fp32():
    """fp32 inputs: agnes_gdn_conv (decode mode) -> agnes_gdn_decode_step -> agnes_gdn_gated_rmsnorm
    keep every intermediate in fp32 too, so the two paths agree to fp32 rounding."""
    rng = np.random.default_rng(330)
    B, hk, hv = 4, 2, 6
    d = _case(rng, B, hk, hv, B, "f32")
    cs1, st1 = dev(d["cs"]), dev(d["st"])
    y1, o1 = _run(d, hk, None, torch.float32, cs1, st1)
    cs2, st2 = dev(d["cs"]), dev(d["st"])
    u = gdn.conv(dev(d["x"]), dev(d["w"]), cu_seqlens=None, conv_state=cs2, l2norm_heads=2 * hk)
    q = u[:, :hk * D].reshape(B, hk, D)
    k = u[:, hk * D:2 * hk * D].reshape(B, hk, D)
    v = u[:, 2 * hk * D:].reshape(B, hv, D)
    o2 = gdn.decode_step(q, k, v, dev(d["g"]), dev(d["beta"]), st2, o_dtype=torch.float32)
    y2 = gdn.gated_rmsnorm(o2, dev(d["z"]), dev(d["nw"]), y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_l2(y1, host(y2)) <= 2e-6 and rel_l2(o1, host(o2)) <= 2e-6
    assert rel_l2(host(st1), host(st2)) <= 2e-6
    np.testing.assert_array_equal(host(cs1), host(cs2))


def test_decode_fused_all_padding_and_empty_batch():
    rng = np.random.default_rng(340)
    d = _case(rng, 3, 1, 3, 2, "bf16")
    cs, st = dev(d["cs"]), dev(d["st"])
    y, o = _run(d, 1, [-1, 2, -5], torch.float32, cs, st)
    assert not y.any() and not o.any()
    np.testing.assert_array_equal(host(cs), d["cs"])
    np.testing.assert_array_equal(host(st), d["st"])
    e = {k: (v[:0] if k in ("x", "g", "beta", "z") else v) for k, v in d.items()}
    y0, _ = _run(e, 1, None, torch.float32, cs, st, want_o=False)
    assert y0.shape == (0, 3, D)


def test_decode_fused_full_size_three_steps():
    """The decode workload's shape: 256 sequences x 16 key / 48 value heads, [256, 10240] inputs,
    805 MB of fp32 states and the bf16 conv cache, three consecutive steps; the oracle follows
    sequences 0, 85, 170, 255 (all heads); every conv-cache row is checked against the shift
    that defines it."""
    cfg = make_config(3)
    picks = [0, 85, 170, 255]
    st = dev(cfg["state"])
    cs = dev(cfg["conv_cache"])
    rst = cfg["state"][picks].astype(np.float64)
    rcs = oracle.as_f64(cfg["conv_cache"][picks])
    prev_cache = cfg["conv_cache"]
    for step in range(3):
        inp = decode_step_inputs(step, gate_input=True)
        y = gdn.decode_fused(dev(inp["x"]), dev(cfg["conv_w"]), cs, dev(inp["g"]), dev(inp["beta"]),
                             dev(inp["z"]), dev(cfg["norm_w"]), st, num_k_heads=16, y_dtype=torch.float32)
        torch.cuda.synchronize()
        ry, _, rcs, rst = oracle.decode_layer_step(
            inp["x"][picks], cfg["conv_w"], rcs, inp["g"][picks], inp["beta"][picks], inp["z"][picks],
            cfg["norm_w"], rst, 16, 48)
        e = rel_l2(host(y)[picks], ry)
        print(f"fused decode step {step}: y rel-L2 {e:.3e}")
        assert e <= 1e-5
        cache = host(cs)
        np.testing.assert_array_equal(cache[..., :2], prev_cache[..., 1:])
        np.testing.assert_array_equal(cache[..., 2], inp["x"])
        prev_cache = cache
    assert rel_l2(host(st)[picks], rst) <= 1e-5
