"""GPU parity of agnes_gdn_layer_prefill (conv + SiLU + L2(q, k), the chunked delta rule and the
gated RMS-norm in one call) against the fp64 oracle of the same composition, with nothing
rounded between the steps.

Tolerances: every output from bf16 inputs (y, o and the final state) is gated at rel-L2 2e-3 on
fp32 outputs.  The norm divides each row by its own RMS: an error common to a row cancels, and
independent errors move the row's RMS only by about e / sqrt(128), so y carries about the
recurrence output's own error (measured: y 4e-4 where o is 3-4e-4).  Against the two-call path
(agnes_gdn_prefill_fused then agnes_gdn_gated_rmsnorm) the recurrence output is the same
arithmetic and must agree bit for bit; y then differs only by the order of the 128-term sum of
squares and the reciprocal square root (a few fp32 ulps), gated at 1e-5 elementwise relative.
A bf16 y is the round-to-nearest-even of the fp32 y of the same inputs, bit for bit.
"""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits, make_config, make_layer_config, LAYER
from tests.helpers import dev, host, rel_l2, as_f64

torch = pytest.importorskip("torch")
import gated_delta_rule_35_amd as gdn  # noqa: E402

pytestmark = pytest.mark.gpu

D = 128
TOL_Y = 2e-3


def _case(rng, lens, hk, hv, hist=True, init=True):
    T = int(sum(lens))
    C = (2 * hk + hv) * D
    f = np.float32
    return dict(
        x=f32_to_bf16_bits(rng.standard_normal((T, C)).astype(f) * f(1.43)),
        w=f32_to_bf16_bits(rng.uniform(-0.5, 0.5, (C, 4)).astype(f)),
        cs=f32_to_bf16_bits(rng.standard_normal((len(lens), C, 3)).astype(f) * f(1.43)) if hist else None,
        g=(-0.05 * np.logaddexp(0, rng.standard_normal((T, hv)))).astype(f),
        beta=(1 / (1 + np.exp(-rng.standard_normal((T, hv))))).astype(f),
        s0=(rng.standard_normal((len(lens), hv, D, D)) * 0.01).astype(f) if init else None,
        z=f32_to_bf16_bits(rng.standard_normal((T, hv, D)).astype(f)),
        nw=f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(D)).astype(f)),
        cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
        hk=hk, hv=hv,
    )


def _layer(d, out_dtype=torch.float32, want_o=False, z_pad=0):
    T, hv = d["g"].shape
    cs = None if d["cs"] is None else dev(d["cs"])
    if z_pad:  # z as a view with a wider token stride
        zb = torch.zeros((T, hv * D + z_pad), dtype=torch.bfloat16, device="cuda")
        zb[:, :hv * D] = dev(d["z"]).view(T, hv * D)
        z = zb[:, :hv * D].view(T, hv, D)
    else:
        z = dev(d["z"])
    o = torch.empty((T, hv, D), dtype=out_dtype, device="cuda") if want_o else None
    y, fin = gdn.layer_prefill(dev(d["x"]), dev(d["w"]), dev(d["g"]), dev(d["beta"]), dev(d["cu"]), z, dev(d["nw"]),
                               num_k_heads=d["hk"], conv_state=cs,
                               initial_state=None if d["s0"] is None else dev(d["s0"]), o=o, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(y), host(fin), (None if cs is None else host(cs)), (None if o is None else host(o))


def _two_calls(d, out_dtype=torch.float32):
    cs = None if d["cs"] is None else dev(d["cs"])
    o, fin = gdn.prefill_fused(dev(d["x"]), dev(d["w"]), dev(d["g"]), dev(d["beta"]), dev(d["cu"]),
                               num_k_heads=d["hk"], conv_state=cs,
                               initial_state=None if d["s0"] is None else dev(d["s0"]), o_dtype=out_dtype)
    y = gdn.gated_rmsnorm(o, dev(d["z"]), dev(d["nw"]))
    torch.cuda.synchronize()
    return host(y), host(fin), host(o)


def _oracle(d):
    ro, rcs, rfin = oracle.prefill_conv_recurrence(d["x"], d["w"], d["cu"], d["cs"], d["g"], d["beta"], d["s0"],
                                                   d["hk"], d["hv"])
    return oracle.gated_rmsnorm(ro, d["z"], d["nw"]), ro, rcs, rfin


def _first128(y, ry, cu):
    rows = np.concatenate([np.arange(a, min(b, a + 128)) for a, b in zip(cu[:-1], cu[1:])])
    return rel_l2(y[rows], ry[rows])


@pytest.mark.parametrize("hist,init,z_pad", [(True, True, 0), (False, False, 64)])
def test_layer_prefill_varlen(hist, init, z_pad):
    """Ragged sequences in one grid: 1 and 2 tokens, an empty one, an exact chunk, partial chunks
    and several chunks; the norm's partial sums cross the value head's four workgroups at every
    chunk, ragged tails included."""
    rng = np.random.default_rng(600 + 2 * hist + init)
    lens = [70, 1, 0, 131, 64, 2, 200]
    d = _case(rng, lens, 2, 6, hist, init)
    y, fin, cs, o = _layer(d, want_o=True, z_pad=z_pad)
    ry, ro, rcs, rfin = _oracle(d)
    ey, ef, eo, ew = rel_l2(y, ry), rel_l2(fin, rfin), rel_l2(o, ro), _first128(y, ry, d["cu"])
    print(f"layer prefill varlen: y {ey:.3e} o {eo:.3e} state {ef:.3e} first-128 {ew:.3e}")
    assert ey <= TOL_Y and ew <= TOL_Y and eo <= 2e-3 and ef <= 2e-3
    if cs is not None:
        np.testing.assert_array_equal(as_f64(cs), rcs)


def test_layer_prefill_equals_two_calls():
    """Same inputs through agnes_gdn_prefill_fused + agnes_gdn_gated_rmsnorm: identical o and final
    state, y within a few fp32 ulps."""
    rng = np.random.default_rng(610)
    d = _case(rng, [100, 64, 9, 300], 2, 6)
    y1, f1, cs1, o1 = _layer(d, want_o=True)
    y2, f2, o2 = _two_calls(d)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)
    rel = np.abs(y1 - y2) / np.maximum(np.abs(y2), 1e-30)
    print(f"layer prefill vs two calls: max rel diff of y {rel.max():.3e}")
    assert float(rel.max()) <= 1e-5


def test_layer_prefill_in_two_stages():
    """Long sequences on a grid that leaves a quarter of the chip free: the call runs as two stages
    (the prep of the second beside the scan of the first, the state carried over in between).
    Ragged lengths split at 13/20 of each sequence's chunks, empty and one-token sequences, conv
    history and initial states; o, the final state and the conv history bit-equal to the two-call
    path, y within a few fp32 ulps of it and within tolerance of the oracle."""
    rng = np.random.default_rng(650)
    lens = [700, 1, 0, 2000, 64, 1300]
    d = _case(rng, lens, 2, 6)
    y1, f1, cs1, o1 = _layer(d, want_o=True)
    cs2 = dev(d["cs"])
    o2, f2 = gdn.prefill_fused(dev(d["x"]), dev(d["w"]), dev(d["g"]), dev(d["beta"]), dev(d["cu"]), num_k_heads=2,
                               conv_state=cs2, initial_state=dev(d["s0"]), o_dtype=torch.float32)
    y2 = gdn.gated_rmsnorm(o2, dev(d["z"]), dev(d["nw"]))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o1, host(o2))
    np.testing.assert_array_equal(f1, host(f2))
    np.testing.assert_array_equal(cs1, host(cs2))
    y2 = host(y2)
    rel = np.abs(y1 - y2) / np.maximum(np.abs(y2), 1e-30)
    ry, _, _, rfin = _oracle(d)
    ey = rel_l2(y1, ry)
    print(f"layer prefill in two stages: max rel diff of y vs two calls {rel.max():.3e}, y vs oracle {ey:.3e}")
    assert float(rel.max()) <= 1e-5 and ey <= TOL_Y and rel_l2(f1, rfin) <= 2e-3



@pytest.mark.parametrize("nstreams", [2, 6])
def test_layer_prefill_in_two_stages_on_several_streams(nstreams):
    """Calls in two stages enqueued back to back on several streams (each with a side stream of its
    own, so the preparations may run at once; six streams are more than the library keeps side
    queues for, so some share one), each call on its own workspace: y, the final states and the
    conv histories equal, bit for bit, the same calls run one after the other on the default
    stream."""
    rng = np.random.default_rng(651)
    lens = [[1500, 900], [1200, 1, 700], [800, 400], [2100], [700, 700, 200], [1000, 999]]  # all in stages
    cases = [_case(rng, lens[i], 2, 6) for i in range(nstreams)]

    def args(d):
        return dict(x=dev(d["x"]), w=dev(d["w"]), g=dev(d["g"]), beta=dev(d["beta"]), cu=dev(d["cu"]),
                    z=dev(d["z"]), nw=dev(d["nw"]), cs=dev(d["cs"]), s0=dev(d["s0"]))

    def call(a, hk):
        return gdn.layer_prefill(a["x"], a["w"], a["g"], a["beta"], a["cu"], a["z"], a["nw"], num_k_heads=hk,
                                 conv_state=a["cs"], initial_state=a["s0"], out_dtype=torch.float32)

    ref = []
    for d in cases:
        a = args(d)
        y, fin = call(a, d["hk"])
        torch.cuda.synchronize()
        ref.append((host(y), host(fin), host(a["cs"])))
    ins = [args(d) for d in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    outs = []
    for a, d, s in zip(ins, cases, streams):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            outs.append(call(a, d["hk"]))
    torch.cuda.synchronize()
    for (y, fin), a, (ry, rf, rc) in zip(outs, ins, ref):
        np.testing.assert_array_equal(host(y), ry)
        np.testing.assert_array_equal(host(fin), rf)
        np.testing.assert_array_equal(host(a["cs"]), rc)


@pytest.mark.parametrize("cuts", [(), (18, 31), (10, 20, 30), (39,), (5, 10, 15, 20, 25, 30, 35)],
                         ids=["one", "three", "four", "late", "eight"])
def test_layer_prefill_stage_cuts_change_nothing(cuts):
    """The stage cuts (agnes_gdn_set_prefill_stages) change the schedule only: one stage, three,
    four, a late single cut and eight stages (middle stages that update the carried state in
    place, and for the short sequences stages with no chunk at all) give y, o, the final state and
    the conv history of the default two stages bit for bit."""
    rng = np.random.default_rng(655)
    d = _case(rng, [700, 1, 0, 2000, 64, 1300], 2, 6)
    ref = _layer(d, want_o=True)
    try:
        gdn.set_prefill_stages(cuts)
        got = _layer(d, want_o=True)
    finally:
        gdn.set_prefill_stages()
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
    again = _layer(d, want_o=True)
    for a, b in zip(again, ref):
        np.testing.assert_array_equal(a, b)

def test_layer_prefill_bf16_outputs_are_rne_of_fp32_outputs():
    rng = np.random.default_rng(620)
    d = _case(rng, [150, 37], 1, 3)
    y32, f32_, _, o32 = _layer(d, want_o=True)
    y16, f16_, _, o16 = _layer(d, torch.bfloat16, want_o=True)
    np.testing.assert_array_equal(y16, f32_to_bf16_bits(y32))
    np.testing.assert_array_equal(o16, f32_to_bf16_bits(o32))
    np.testing.assert_array_equal(f16_, f32_)


def test_layer_prefill_grid_larger_than_the_chip():
    """Three sequences of the 48-value-head layer need 576 workgroups, more than the chip holds at
    once: heads whose workgroups start late wait for earlier ones to finish, and every row still
    gets its four partial sums (a late partner, a ragged tail, a one-token sequence)."""
    rng = np.random.default_rng(630)
    d = _case(rng, [70, 5, 1], LAYER["num_k_heads"], LAYER["num_v_heads"])
    y, fin, cs, _ = _layer(d)
    ry, _, rcs, rfin = _oracle(d)
    ey, ef = rel_l2(y, ry), rel_l2(fin, rfin)
    print(f"layer prefill, 576 workgroups: y {ey:.3e} state {ef:.3e}")
    assert ey <= TOL_Y and ef <= 2e-3
    np.testing.assert_array_equal(as_f64(cs), rcs)


def test_layer_prefill_repeated_calls_reuse_the_workspace():
    """The same workspace twice in a row (the exchange words and the ticket counter of the first
    call are cleared by the second) and a different batch in between."""
    rng = np.random.default_rng(640)
    d1 = _case(rng, [130, 64], 2, 6)
    d2 = _case(rng, [7, 200, 3], 2, 6)
    ws = torch.empty(gdn.layer_prefill_workspace_size(3, 210, 2, 6), dtype=torch.uint8, device="cuda")
    outs = []
    for d in (d1, d2, d1):
        T = d["g"].shape[0]
        y, _ = gdn.layer_prefill(dev(d["x"]), dev(d["w"]), dev(d["g"]), dev(d["beta"]), dev(d["cu"]), dev(d["z"]),
                                 dev(d["nw"]), num_k_heads=2, conv_state=dev(d["cs"]), initial_state=dev(d["s0"]),
                                 out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        outs.append(host(y))
    np.testing.assert_array_equal(outs[0], outs[2])
    ry, _, _, _ = _oracle(d2)
    assert rel_l2(outs[1], ry) <= TOL_Y


def test_layer_prefill_all_sequences_empty_after_a_full_call():
    """A batch of empty sequences (y may then be null) right after a call that left its role
    counters and exchange words in the same workspace, the rest of which holds all-ones bytes:
    the empty call still clears its own counters, nothing is written to y, the final states are
    the initial ones, the conv history is unchanged and no error bit is set."""
    rng = np.random.default_rng(660)
    d1 = _case(rng, [150, 40], 2, 6)
    ws = torch.empty(gdn.layer_prefill_workspace_size(3, 190, 2, 6), dtype=torch.uint8, device="cuda")
    ws.fill_(255)  # every word the empty call would find uncleared reads as a huge counter
    gdn.layer_prefill(dev(d1["x"]), dev(d1["w"]), dev(d1["g"]), dev(d1["beta"]), dev(d1["cu"]), dev(d1["z"]),
                      dev(d1["nw"]), num_k_heads=2, conv_state=dev(d1["cs"]), initial_state=dev(d1["s0"]),
                      out_dtype=torch.float32, workspace=ws)
    d0 = _case(rng, [0, 0, 0], 2, 6)
    cs = dev(d0["cs"])
    y = torch.full((0, 6, D), 7.0, dtype=torch.float32, device="cuda")
    y0, fin = gdn.layer_prefill(dev(d0["x"]), dev(d0["w"]), dev(d0["g"]), dev(d0["beta"]), dev(d0["cu"]),
                                dev(d0["z"]), dev(d0["nw"]), num_k_heads=2, conv_state=cs,
                                initial_state=dev(d0["s0"]), y=y, workspace=ws)
    torch.cuda.synchronize()
    assert gdn.workspace_status(ws) == 0
    assert y0.shape == (0, 6, D)
    np.testing.assert_array_equal(host(fin), d0["s0"])
    np.testing.assert_array_equal(host(cs), d0["cs"])


def test_layer_prefill_in_a_graph():
    """The two-stage call (one 1024-token sequence on 2 key / 6 value heads) captured into a graph
    with its side stream, replayed three times with eager work on the stream in between: every
    replay equals the eager call bit for bit."""
    rng = np.random.default_rng(670)
    d = _case(rng, [1024], 2, 6, hist=False)
    x, w, g, be, cu, z, nw, s0 = (dev(d[k]) for k in ("x", "w", "g", "beta", "cu", "z", "nw", "s0"))
    ws = torch.empty(gdn.layer_prefill_workspace_size(1, 1024, 2, 6), dtype=torch.uint8, device="cuda")
    y_ref, f_ref = gdn.layer_prefill(x, w, g, be, cu, z, nw, num_k_heads=2, initial_state=s0, out_dtype=torch.float32,
                                     workspace=ws)
    torch.cuda.synchronize()
    y_ref, f_ref = host(y_ref), host(f_ref)
    y = torch.empty((1024, 6, D), dtype=torch.float32, device="cuda")
    fin = torch.empty((1, 6, D, D), dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # capture on a non-default stream, as torch requires
        with torch.cuda.graph(graph):
            gdn.layer_prefill(x, w, g, be, cu, z, nw, num_k_heads=2, initial_state=s0, final_state=fin, y=y,
                              workspace=ws)
    torch.cuda.synchronize()
    for r in range(3):
        y.fill_(float("nan"))
        fin.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda") * 2.0  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), y_ref)
        np.testing.assert_array_equal(host(fin), f_ref)
        del junk


def test_layer_prefill_full_layer_t8192():
    """The layer's prefill workload (T = 8192, 16 key / 48 value heads, bf16 projection x, gate z
    and norm weight of the chain workload) in the launch configuration the benchmark times (two
    stages, roles claimed per XCD range); the oracle follows all 48 value heads, so every key
    group and every one of the eight role ranges is checked."""
    cfg = make_config(1)
    T, HK, HV = 8192, LAYER["num_k_heads"], LAYER["num_v_heads"]
    cu = cfg["cu_seqlens"]
    y, fin = gdn.layer_prefill(dev(cfg["x"]), dev(cfg["conv_w"]), dev(cfg["g"]), dev(cfg["beta"]), dev(cu),
                               dev(cfg["z"]), dev(cfg["norm_w"]), num_k_heads=HK, out_dtype=torch.float32)
    torch.cuda.synchronize()
    y, fin = host(y), host(fin)
    u, _ = oracle.causal_conv(cfg["x"], cfg["conv_w"], cu, None, l2_heads=2 * HK)
    q, k, v = u[:, :HK * D].reshape(T, HK, D), u[:, HK * D:2 * HK * D].reshape(T, HK, D), u[:, 2 * HK * D:].reshape(T, HV, D)
    del u
    ro, rf = oracle.recurrence(q, k, v, cfg["g"], cfg["beta"], cu)
    ry = oracle.gated_rmsnorm(ro, cfg["z"], cfg["norm_w"])
    ey, ef = rel_l2(y, ry), rel_l2(fin, rf)
    worst = max(rel_l2(y[:, h], ry[:, h]) for h in range(HV))
    print(f"layer prefill T=8192 rel-L2 y={ey:.3e} state={ef:.3e} worst head y={worst:.3e}")
    assert ey <= TOL_Y and ef <= 2e-3 and worst <= TOL_Y


# value heads the oracle follows at the long and varlen sizes: stride 5 covers all three positions
# of a key group (0, 5, 10 -> 0, 2, 1 mod 3) and 10 of the 16 key groups
HEADS10 = list(range(0, 48, 5))


def _sub_layer(d, heads, a, b, with_s0=True):
    """The oracle of the whole layer on tokens [a, b) of one sequence (which starts at a), on the
    value heads ``heads`` only: each head is taken with its key head's q and k channels as a
    layer of len(heads) key and value heads (conv and L2 act per channel and per head)."""
    kh = [h // 3 for h in heads]
    ch = np.concatenate([np.arange(128 * j, 128 * j + 128) for j in kh]
                        + [np.arange(2048 + 128 * j, 2048 + 128 * j + 128) for j in kh]
                        + [np.arange(4096 + 128 * h, 4096 + 128 * h + 128) for h in heads])
    x = np.ascontiguousarray(d["x"][a:b][:, ch])
    w = np.ascontiguousarray(d["conv_w"][ch])
    s0 = d["s0n"][:, heads] if with_s0 and d.get("s0n") is not None else None
    n = len(heads)
    ro, _, rf = oracle.prefill_conv_recurrence(x, w, np.array([0, b - a]), None, d["g"][a:b][:, heads],
                                               d["beta"][a:b][:, heads], s0, n, n)
    ry = oracle.gated_rmsnorm(ro, np.ascontiguousarray(d["z"][a:b][:, heads]), d["norm_w"])
    return ry, rf[0]


def _run_layer_big(d):
    """The whole-layer call on a large workload; y stays on the device (fp32) for sampling."""
    s0 = d["initial_state"]
    y, fin = gdn.layer_prefill(dev(d["x"]), dev(d["conv_w"]), dev(d["g"]), dev(d["beta"]), dev(d["cu_seqlens"]),
                               dev(d["z"]), dev(d["norm_w"]), num_k_heads=LAYER["num_k_heads"],
                               initial_state=None if s0 is None else dev(s0), out_dtype=torch.float32)
    torch.cuda.synchronize()
    return y, host(fin)


def test_layer_prefill_long_t65536():
    """One sequence of 65536 tokens (1024 chunks, split at 13/20 between the two stages) with an
    initial state, through the whole-layer call; the oracle follows value heads 0, 5, .., 45 over
    the whole sequence, and the first 128 tokens (where the initial state still dominates) are
    gated on their own."""
    d = make_layer_config(2)
    yd, fin = _run_layer_big(d)
    y = host(yd[:, HEADS10])
    del yd
    d["s0n"] = d["initial_state"][0][None]
    T = d["x"].shape[0]
    ry, rf = _sub_layer(d, HEADS10, 0, T)
    ey, ef, ew = rel_l2(y, ry), rel_l2(fin[0, HEADS10], rf), rel_l2(y[:128], ry[:128])
    print(f"layer prefill T=65536 rel-L2 y={ey:.3e} state={ef:.3e} first-128 y={ew:.3e}")
    assert ey <= TOL_Y and ef <= 2e-3 and ew <= TOL_Y


def test_layer_prefill_varlen_32_sequences():
    """The 32-sequence log-uniform batch (251,984 tokens, 1536 value-head chains, more workgroups
    than the chip holds) through the whole-layer call: the first 128 tokens of every sequence on
    value heads 0, 5, .., 45, and four whole sequences (the shortest, the longest, the first two)
    with their final states."""
    d = make_layer_config(4)
    cu = d["cu_seqlens"]
    lens = np.diff(cu)
    yd, fin = _run_layer_big(d)
    rows = np.concatenate([np.arange(a, min(b, a + 128)) for a, b in zip(cu[:-1], cu[1:])])
    yw = host(yd[torch.from_numpy(rows).cuda()][:, HEADS10])
    worst = 0.0
    off = 0
    for n in range(len(lens)):
        a, m = int(cu[n]), int(min(lens[n], 128))
        d["s0n"] = d["initial_state"][n][None]
        ry, _ = _sub_layer(d, HEADS10, a, a + m)
        worst = max(worst, rel_l2(yw[off:off + m], ry))
        off += m
    print(f"varlen layer prefill: worst first-128 window y rel-L2 {worst:.3e}")
    assert worst <= TOL_Y
    for n in sorted({0, 1, int(np.argmin(lens)), int(np.argmax(lens))}):
        a, b = int(cu[n]), int(cu[n + 1])
        d["s0n"] = d["initial_state"][n][None]
        y = host(yd[a:b][:, HEADS10])
        ry, rf = _sub_layer(d, HEADS10, a, b)
        ey, ef = rel_l2(y, ry), rel_l2(fin[n, HEADS10], rf)
        print(f"seq {n} len {b - a}: y rel-L2 {ey:.3e} state {ef:.3e}")
        assert ey <= TOL_Y and ef <= 2e-3
