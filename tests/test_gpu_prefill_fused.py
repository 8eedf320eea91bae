"""GPU parity of agnes_gdn_prefill_fused (conv + SiLU + L2(q, k) and the chunked prefill in one
call, from the raw q|k|v projection) against the fp64 oracle of the same composition, with nothing
rounded between the conv and the recurrence.

Tolerances: rel-L2 2e-3 on an fp32 `o` and on the final states (the matrix-core operands are fp16,
as for agnes_gdn_prefill_chunked); the bf16 `o` of the same call must be the round-to-nearest-even
of the fp32 `o`, bit for bit; the final conv history is a copy of input values and must match
exactly.  Sequences are gated on their first 128 tokens as well, where a wrong conv history or
initial state would show.
"""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits, make_config, LAYER
from tests.helpers import dev, host, rel_l2

torch = pytest.importorskip("torch")
import gated_delta_rule_35_amd as gdn  # noqa: E402

pytestmark = pytest.mark.gpu

D = 128


def _case(rng, lens, hk, hv, hist=True, init=True, bias=False):
    T = int(sum(lens))
    C = (2 * hk + hv) * D
    f = np.float32
    return dict(
        x=f32_to_bf16_bits(rng.standard_normal((T, C)).astype(f) * f(1.43)),
        w=f32_to_bf16_bits(rng.uniform(-0.5, 0.5, (C, 4)).astype(f)),
        b=f32_to_bf16_bits(rng.uniform(-0.2, 0.2, C).astype(f)) if bias else None,
        cs=f32_to_bf16_bits(rng.standard_normal((len(lens), C, 3)).astype(f) * f(1.43)) if hist else None,
        g=(-0.05 * np.logaddexp(0, rng.standard_normal((T, hv)))).astype(f),
        beta=(1 / (1 + np.exp(-rng.standard_normal((T, hv))))).astype(f),
        s0=(rng.standard_normal((len(lens), hv, D, D)) * 0.01).astype(f) if init else None,
        cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
        hk=hk, hv=hv,
    )


def _run(d, o_dtype=torch.float32):
    cs = None if d["cs"] is None else dev(d["cs"])
    o, fin = gdn.prefill_fused(dev(d["x"]), dev(d["w"]), dev(d["g"]), dev(d["beta"]), dev(d["cu"]),
                               num_k_heads=d["hk"], conv_bias=None if d["b"] is None else dev(d["b"]),
                               conv_state=cs, initial_state=None if d["s0"] is None else dev(d["s0"]),
                               o_dtype=o_dtype)
    torch.cuda.synchronize()
    return host(o), host(fin), (None if cs is None else host(cs))


def _oracle(d):
    return oracle.prefill_conv_recurrence(d["x"], d["w"], d["cu"], d["cs"], d["g"], d["beta"], d["s0"], d["hk"],
                                          d["hv"], conv_bias=d["b"])


def _first128(o, ro, cu):
    rows = np.concatenate([np.arange(a, min(b, a + 128)) for a, b in zip(cu[:-1], cu[1:])])
    return rel_l2(o[rows], ro[rows])


@pytest.mark.parametrize("hist,init,bias", [(True, True, False), (False, False, True), (True, False, True)])
def test_prefill_fused_varlen(hist, init, bias):
    """Ragged sequences: 1 and 2 tokens (shorter than the conv halo), an empty one, an exact
    chunk, partial chunks and several chunks."""
    rng = np.random.default_rng(400 + 4 * hist + 2 * init + bias)
    lens = [70, 1, 0, 131, 64, 2, 200]
    d = _case(rng, lens, 2, 6, hist, init, bias)
    o, fin, cs = _run(d)
    ro, rcs, rfin = _oracle(d)
    eo, ef, ew = rel_l2(o, ro), rel_l2(fin, rfin), _first128(o, ro, d["cu"])
    print(f"fused prefill varlen: o {eo:.3e} state {ef:.3e} first-128 {ew:.3e}")
    assert eo <= 2e-3 and ef <= 2e-3 and ew <= 2e-3
    if cs is not None:
        np.testing.assert_array_equal(oracle.as_f64(cs), rcs)


def test_prefill_fused_two_stages_equal_one():
    """A long sequence on a grid that leaves a quarter of the chip free runs in two stages (the
    second half's prep beside the first half's scan); the same sequence followed by 8 empty ones
    fills the grid past that and runs in one.  o, the final state and the conv history agree
    bit for bit."""
    rng = np.random.default_rng(430)
    d = _case(rng, [2000], 2, 6)
    o1, f1, cs1 = _run(d)
    d9 = dict(d, cu=np.concatenate([d["cu"], np.full(8, d["cu"][-1])]).astype(np.int32),
              cs=np.concatenate([d["cs"], np.zeros((8,) + d["cs"].shape[1:], np.uint16)]),
              s0=np.concatenate([d["s0"], np.zeros((8,) + d["s0"].shape[1:], np.float32)]))
    o9, f9, cs9 = _run(d9)
    np.testing.assert_array_equal(o1, o9)
    np.testing.assert_array_equal(f1[0], f9[0])
    np.testing.assert_array_equal(cs1[0], cs9[0])


def test_prefill_fused_bf16_output_is_rne_of_fp32_output():
    rng = np.random.default_rng(410)
    d = _case(rng, [150, 37], 1, 3)
    o32, f32_, _ = _run(d)
    o16, f16_, _ = _run(d, torch.bfloat16)
    np.testing.assert_array_equal(o16, f32_to_bf16_bits(o32))
    np.testing.assert_array_equal(f16_, f32_)


def test_prefill_fused_close_to_separate_calls():
    """agnes_gdn_conv -> agnes_gdn_prefill_chunked computes the same layer with q, k, v stored in
    bf16 in between; the two agree to that rounding (~1e-3)."""
    rng = np.random.default_rng(420)
    d = _case(rng, [100, 64, 9], 2, 6)
    o1, f1, cs1 = _run(d)
    cs2 = dev(d["cs"])
    y = gdn.conv(dev(d["x"]), dev(d["w"]), cu_seqlens=dev(d["cu"]), conv_state=cs2, l2norm_heads=4)
    T = y.shape[0]
    o2, f2 = gdn.prefill_chunked(y[:, :256].view(T, 2, D), y[:, 256:512].view(T, 2, D), y[:, 512:].view(T, 6, D),
                                 dev(d["g"]), dev(d["beta"]), dev(d["cu"]), initial_state=dev(d["s0"]),
                                 o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_l2(o1, host(o2)) <= 4e-3 and rel_l2(f1, host(f2)) <= 4e-3
    np.testing.assert_array_equal(cs1, host(cs2))


def test_prefill_fused_full_layer_t8192():
    """The layer's prefill workload (T = 8192, 16 key / 48 value heads, x = the bf16 projection of
    the chain workload); the oracle follows all 48 value heads."""
    cfg = make_config(1)
    T, HK, HV = 8192, LAYER["num_k_heads"], LAYER["num_v_heads"]
    cu = cfg["cu_seqlens"]
    o, fin = gdn.prefill_fused(dev(cfg["x"]), dev(cfg["conv_w"]), dev(cfg["g"]), dev(cfg["beta"]), dev(cu),
                               num_k_heads=HK, o_dtype=torch.float32)
    torch.cuda.synchronize()
    o, fin = host(o), host(fin)
    u, _ = oracle.causal_conv(cfg["x"], cfg["conv_w"], cu, None, l2_heads=2 * HK)
    q, k, v = u[:, :HK * D].reshape(T, HK, D), u[:, HK * D:2 * HK * D].reshape(T, HK, D), u[:, 2 * HK * D:].reshape(T, HV, D)
    del u
    ro, rf = oracle.recurrence(q, k, v, cfg["g"], cfg["beta"], cu)
    eo, ef = rel_l2(o, ro), rel_l2(fin, rf)
    worst = max(rel_l2(o[:, h], ro[:, h]) for h in range(HV))
    print(f"fused prefill T=8192 rel-L2 o={eo:.3e} state={ef:.3e} worst head o={worst:.3e}")
    assert eo <= 2e-3 and ef <= 2e-3 and worst <= 2e-3
