"""GPU parity of every C-ABI call against the fp64 oracle on identical input bytes.

Shapes span several 64-token chunks and ragged tails; tolerances (rel-L2 against fp64):
  * bf16-input recurrence (fp16 matrix-core operands, fp32 state): 2e-3, on an fp32 `o`;
    the bf16 `o` of the same call must be the round-to-nearest-even of the fp32 `o`, bit for bit;
  * fp32-input recurrence and every decode step (fp32 arithmetic throughout): 1e-5;
  * conv / gated RMSNorm with bf16 outputs: bit-exact (the correctly rounded fp64 value) for
    >= 99.9 % of elements and within 1 bf16 ulp elsewhere, except where a near-cancelling fp32
    sum of the 4 conv taps leaves an absolute error <= 1e-5 (CONV_ABS_TOL); fp32 outputs: 1e-6.
"""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits, unit_vectors
from synth.configs import sequence_inputs, make_config
from tests.helpers import dev, host, rel_l2, bf16_ulps, check_bf16_out

# fp32 sum of 4 conv taps (|w| <= 1/2, |x| < 8): rounding error <= 16 * 4 * 2^-24 ~ 4e-6 before
# SiLU (slope <= 1.1) and the L2 scaling; near-cancelling sums are exact only to this absolute level.
CONV_ABS_TOL = 1e-5

torch = pytest.importorskip("torch")
import gated_delta_rule_35_amd as gdn  # noqa: E402

pytestmark = pytest.mark.gpu


def _t(a):
    return dev(a)


def run_prefill(s, o_dtype=torch.float32, final=True, scale=1.0, initial=True):
    cu = _t(s["cu_seqlens"])
    s0 = _t(s["initial_state"]) if (initial and s["initial_state"] is not None) else None
    o, fin = gdn.prefill_chunked(_t(s["q"]), _t(s["k"]), _t(s["v"]), _t(s["g"]), _t(s["beta"]), cu,
                                 initial_state=s0, output_final_state=final, o_dtype=o_dtype, scale=scale)
    torch.cuda.synchronize()
    return host(o), (host(fin) if fin is not None else None)


def oracle_prefill(s, scale=1.0):
    return oracle.recurrence(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu_seqlens"], s["initial_state"],
                             scale=scale)


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("B,hk,hv,dtype", [(5, 2, 6, "bf16"), (3, 16, 48, "bf16"), (4, 1, 3, "f32")])
def test_decode_step_matches_oracle(B, hk, hv, dtype):
    rng = np.random.default_rng(100 + B)
    s = sequence_inputs(rng, [1] * B, hk, hv, 128, dtype=dtype, init="normal", init_std=0.3)
    st = _t(s["initial_state"])
    o = gdn.decode_step(_t(s["q"]), _t(s["k"]), _t(s["v"]), _t(s["g"]), _t(s["beta"]), st,
                        o_dtype=torch.float32, scale=0.7)
    torch.cuda.synchronize()
    ro, rs = oracle.decode_step(s["q"], s["k"], s["v"], s["g"], s["beta"], s["initial_state"], scale=0.7)
    assert rel_l2(host(o), ro) <= 1e-5
    assert rel_l2(host(st), rs) <= 1e-5
    # bf16 output of the same step is the RNE of the fp32 output
    st2 = _t(s["initial_state"])
    ob = gdn.decode_step(_t(s["q"]), _t(s["k"]), _t(s["v"]), _t(s["g"]), _t(s["beta"]), st2,
                         o_dtype=torch.bfloat16, scale=0.7)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ob), f32_to_bf16_bits(host(o)))
    np.testing.assert_array_equal(host(st2), host(st))


def test_decode_step_reads_strided_conv_output_views():
    """q/k/v as views into one [B, 10240] conv-output row (token stride 10240)."""
    rng = np.random.default_rng(11)
    B = 6
    y = f32_to_bf16_bits(rng.standard_normal((B, 10240)).astype(np.float32) * 0.1)
    q, k, v = y[:, :2048].reshape(B, 16, 128), y[:, 2048:4096].reshape(B, 16, 128), y[:, 4096:].reshape(B, 48, 128)
    g = (-0.05 * rng.random((B, 48))).astype(np.float32)
    beta = rng.random((B, 48)).astype(np.float32)
    s0 = (rng.standard_normal((B, 48, 128, 128)) * 0.01).astype(np.float32)
    yt = _t(y)
    st = _t(s0)
    o = gdn.decode_step(yt[:, :2048].view(B, 16, 128), yt[:, 2048:4096].view(B, 16, 128),
                        yt[:, 4096:].view(B, 48, 128), _t(g), _t(beta), st, o_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = oracle.decode_step(q, k, v, g, beta, s0)
    assert rel_l2(host(o), ro) <= 1e-5 and rel_l2(host(st), rs) <= 1e-5


# ------------------------------------------------------------------ conv

def _conv_case(rng, lens, C, dtype, with_state, l2):
    T = sum(lens)
    x = rng.standard_normal((T, C)).astype(np.float32) * 1.4
    w = rng.uniform(-0.5, 0.5, (C, 4)).astype(np.float32)
    st = rng.standard_normal((len(lens), C, 3)).astype(np.float32) if with_state else None
    conv = f32_to_bf16_bits if dtype == "bf16" else (lambda a: a)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return conv(x), conv(w), (conv(st) if st is not None else None), cu


def _check_bf16_out(gpu_bits, ref, abs_tol=CONV_ABS_TOL):
    check_bf16_out(gpu_bits, ref, abs_tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("with_state", [True, False])
def test_conv_prefill_varlen(dtype, with_state):
    rng = np.random.default_rng(21)
    lens = [1, 2, 0, 70, 3, 129, 17]
    C = 1024
    x, w, st, cu = _conv_case(rng, lens, C, dtype, with_state, 4)
    stt = _t(st) if st is not None else None
    y = gdn.conv(_t(x), _t(w), cu_seqlens=_t(cu), conv_state=stt, l2norm_heads=4)
    torch.cuda.synchronize()
    ry, rst = oracle.causal_conv(x, w, cu, st, l2_heads=4)
    if dtype == "bf16":
        _check_bf16_out(host(y), ry)
    else:
        assert rel_l2(host(y), ry) <= 1e-6
    if st is not None:
        np.testing.assert_array_equal(oracle.as_f64(host(stt)), rst)  # history is a copy: exact


def test_conv_prefill_strided_rows_and_tail():
    """x as a column slice of a wider buffer (row stride 1536), T not a multiple of 16."""
    rng = np.random.default_rng(22)
    T, C = 333, 1024
    big = f32_to_bf16_bits(rng.standard_normal((T, 1536)).astype(np.float32))
    w = f32_to_bf16_bits(rng.uniform(-0.5, 0.5, (C, 4)).astype(np.float32))
    cu = np.array([0, T], np.int32)
    bt = _t(big)
    y = gdn.conv(bt[:, 256:256 + C], _t(w), cu_seqlens=_t(cu), l2norm_heads=2)
    torch.cuda.synchronize()
    ry, _ = oracle.causal_conv(big[:, 256:256 + C], w, cu, None, l2_heads=2)
    _check_bf16_out(host(y), ry)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_decode_mode(dtype):
    rng = np.random.default_rng(23)
    N, C = 9, 2048
    x, w, st, _ = _conv_case(rng, [1] * N, C, dtype, True, 8)
    stt = _t(st)
    y = gdn.conv(_t(x), _t(w), cu_seqlens=None, conv_state=stt, l2norm_heads=8)
    torch.cuda.synchronize()
    ry, rst = oracle.causal_conv(x, w, np.arange(N + 1), st, l2_heads=8)
    if dtype == "bf16":
        _check_bf16_out(host(y), ry)
    else:
        assert rel_l2(host(y), ry) <= 1e-6
    np.testing.assert_array_equal(oracle.as_f64(host(stt)), rst)


def _at_4_bytes(t):
    """A copy of t whose data starts 4 bytes past a 16-byte boundary (the C ABI's minimum for the
    conv's taps, bias and history)."""
    off = 4 // t.element_size()
    buf = torch.empty(t.numel() + off, dtype=t.dtype, device=t.device)
    v = buf[off:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 == 4
    return v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_conv_params_at_4_byte_alignment(dtype, mode):
    """Taps, bias and history 16-byte aligned are read and written as 16-byte vectors, at the C
    ABI's 4-byte minimum one element at a time: the outputs and the advanced history agree bit for
    bit, and with the oracle."""
    rng = np.random.default_rng(24)
    lens = [1] * 9 if mode == "decode" else [5, 1, 0, 70, 2]
    C = 2048
    x, w, st, cu = _conv_case(rng, lens, C, dtype, True, 8)
    conv = f32_to_bf16_bits if dtype == "bf16" else (lambda a: a)
    b = conv(rng.uniform(-0.5, 0.5, C).astype(np.float32))
    cut = None if mode == "decode" else _t(cu)
    outs = []
    for place in (lambda t: t, _at_4_bytes):
        wt, bt, stt = place(_t(w)), place(_t(b)), place(_t(st))
        y = gdn.conv(_t(x), wt, bias=bt, cu_seqlens=cut, conv_state=stt, l2norm_heads=8)
        torch.cuda.synchronize()
        outs.append((host(y), host(stt)))
    np.testing.assert_array_equal(outs[1][0], outs[0][0])
    np.testing.assert_array_equal(outs[1][1], outs[0][1])
    ry, rst = oracle.causal_conv(x, w, cu, st, l2_heads=8, bias=b)
    if dtype == "bf16":
        _check_bf16_out(outs[0][0], ry)
    else:
        assert rel_l2(outs[0][0], ry) <= 1e-6
    np.testing.assert_array_equal(oracle.as_f64(outs[0][1]), rst)


# ------------------------------------------------------------------ gated RMSNorm

@pytest.mark.parametrize("odt,zdt,ydt", [("bf16", "bf16", "bf16"), ("f32", "bf16", "bf16"),
                                         ("f32", "f32", "f32"), ("bf16", "f32", "f32")])
def test_gated_rmsnorm(odt, zdt, ydt):
    rng = np.random.default_rng(31)
    rows = 1000  # not a multiple of the 64 rows per block
    cvt = {"bf16": f32_to_bf16_bits, "f32": lambda a: a.astype(np.float32)}
    o = cvt[odt](rng.standard_normal((rows, 128)).astype(np.float32) * 3)
    z = cvt[zdt](rng.standard_normal((rows, 128)).astype(np.float32))
    w = cvt[zdt]((1 + 0.1 * rng.standard_normal(128)).astype(np.float32))
    y = gdn.gated_rmsnorm(_t(o), _t(z), _t(w), y_dtype=torch.bfloat16 if ydt == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ry = oracle.gated_rmsnorm(o, z, w)
    if ydt == "bf16":
        _check_bf16_out(host(y), ry)
    else:
        assert rel_l2(host(y), ry) <= 1e-6


def test_gated_rmsnorm_in_place():
    rng = np.random.default_rng(32)
    o = f32_to_bf16_bits(rng.standard_normal((200, 128)).astype(np.float32))
    z = f32_to_bf16_bits(rng.standard_normal((200, 128)).astype(np.float32))
    w = f32_to_bf16_bits(np.ones(128, np.float32))
    ot = _t(o)
    y = gdn.gated_rmsnorm(ot, _t(z), _t(w), y=ot)
    torch.cuda.synchronize()
    _check_bf16_out(host(y), oracle.gated_rmsnorm(o, z, w))


# ------------------------------------------------------------------ prefill, fp32 inputs

def test_prefill_fp32_config0():
    """Single key group, fp32 inputs, T = 512: rel-L2 <= 1e-5 on o and the final state."""
    s = make_config(0)
    o, fin = run_prefill(s)
    ro, rf = oracle_prefill(s)
    assert rel_l2(o, ro) <= 1e-5
    assert rel_l2(fin, rf) <= 1e-5


@pytest.mark.parametrize("lens", [[1], [63], [65, 0, 130], [0, 0], [200, 1, 64]])
def test_prefill_fp32_lengths(lens):
    rng = np.random.default_rng(sum(lens) + 3)
    s = sequence_inputs(rng, lens, 2, 6, 128, dtype="f32", init="alternate", init_std=0.1)
    o, fin = run_prefill(s, scale=0.5)
    ro, rf = oracle_prefill(s, scale=0.5)
    if sum(lens):
        assert rel_l2(o, ro) <= 1e-5
    assert rel_l2(fin, rf) <= 1e-5


# ------------------------------------------------------------------ prefill, bf16 inputs

@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 128, 129, 300])
def test_prefill_bf16_lengths(T):
    rng = np.random.default_rng(T)
    s = sequence_inputs(rng, [T], 2, 6, 128, dtype="bf16", init="normal")
    o, fin = run_prefill(s)
    ro, rf = oracle_prefill(s)
    eo, ef = rel_l2(o, ro), rel_l2(fin, rf)
    print(f"T={T} rel-L2 o={eo:.3e} state={ef:.3e}")
    assert eo <= 2e-3 and ef <= 2e-3


def test_prefill_bf16_varlen_full_heads():
    rng = np.random.default_rng(41)
    s = sequence_inputs(rng, [0, 5, 64, 0, 200, 1, 97], 16, 48, 128, dtype="bf16", init="alternate")
    o, fin = run_prefill(s)
    ro, rf = oracle_prefill(s)
    eo, ef = rel_l2(o, ro), rel_l2(fin, rf)
    print(f"varlen rel-L2 o={eo:.3e} state={ef:.3e}")
    assert eo <= 2e-3 and ef <= 2e-3
    # zero-length sequences pass their initial state through unchanged
    np.testing.assert_array_equal(fin[0], s["initial_state"][0])
    np.testing.assert_array_equal(fin[3], s["initial_state"][3])


def test_prefill_many_sequences():
    """300 sequences (more than one per thread of the chunk-offset prefix sum), lengths 0..60:
    every sequence's output and final state, including empty ones passing their state through."""
    rng = np.random.default_rng(46)
    lens = [int(x) for x in rng.integers(0, 61, size=300)]
    lens[0], lens[1], lens[299] = 0, 64, 129
    s = sequence_inputs(rng, lens, 1, 3, 128, dtype="bf16", init="normal")
    o, fin = run_prefill(s)
    ro, rf = oracle_prefill(s)
    eo, ef = rel_l2(o, ro), rel_l2(fin, rf)
    print(f"300 sequences rel-L2 o={eo:.3e} state={ef:.3e}")
    assert eo <= 2e-3 and ef <= 2e-3
    np.testing.assert_array_equal(fin[0], s["initial_state"][0])


def test_prefill_two_stages_equal_one():
    """As for the fused call: one 2000-token sequence (two stages) against the same sequence
    followed by 8 empty ones (one stage): o and the final state bit for bit."""
    rng = np.random.default_rng(47)
    s1 = sequence_inputs(rng, [2000], 2, 6, 128, dtype="bf16", init="normal")
    s9 = dict(s1, cu_seqlens=np.concatenate([s1["cu_seqlens"], np.full(8, 2000)]).astype(np.int32),
              initial_state=np.concatenate([s1["initial_state"], np.zeros((8, 6, 128, 128), np.float32)]))
    o1, f1 = run_prefill(s1)
    o9, f9 = run_prefill(s9)
    np.testing.assert_array_equal(o1, o9)
    np.testing.assert_array_equal(f1[0], f9[0])


def test_prefill_bf16_output_is_rne_of_fp32_output():
    rng = np.random.default_rng(42)
    s = sequence_inputs(rng, [150, 70], 2, 6, 128, dtype="bf16", init="normal")
    o32, f32_ = run_prefill(s, torch.float32)
    o16, f16_ = run_prefill(s, torch.bfloat16)
    np.testing.assert_array_equal(o16, f32_to_bf16_bits(o32))
    np.testing.assert_array_equal(f16_, f32_)


def test_prefill_deterministic_null_state_and_in_place():
    rng = np.random.default_rng(43)
    s = sequence_inputs(rng, [190], 2, 6, 128, dtype="bf16", init="zeros")
    a_o, a_f = run_prefill(s)
    b_o, b_f = run_prefill(s)
    np.testing.assert_array_equal(a_o, b_o)          # run twice: bit-identical
    np.testing.assert_array_equal(a_f, b_f)
    n_o, n_f = run_prefill(s, initial=False)          # NULL initial state == explicit zeros
    np.testing.assert_array_equal(n_o, a_o)
    np.testing.assert_array_equal(n_f, a_f)
    s2 = sequence_inputs(rng, [130], 2, 6, 128, dtype="bf16", init="normal")
    ref_o, ref_f = run_prefill(s2)
    st = _t(s2["initial_state"])                      # final_state aliases initial_state
    o, _ = gdn.prefill_chunked(_t(s2["q"]), _t(s2["k"]), _t(s2["v"]), _t(s2["g"]), _t(s2["beta"]),
                               _t(s2["cu_seqlens"]), initial_state=st, final_state=st, o_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o), ref_o)
    np.testing.assert_array_equal(host(st), ref_f)


def test_prefill_packed_equals_separate_bit_exact():
    rng = np.random.default_rng(44)
    lens = [70, 129, 1, 64]
    s = sequence_inputs(rng, lens, 2, 6, 128, dtype="bf16", init="normal")
    o, fin = run_prefill(s)
    cu = s["cu_seqlens"]
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        part = dict(s, q=s["q"][a:b], k=s["k"][a:b], v=s["v"][a:b], g=s["g"][a:b], beta=s["beta"][a:b],
                    cu_seqlens=np.array([0, b - a], np.int32), initial_state=s["initial_state"][n:n + 1])
        po, pf = run_prefill(part)
        np.testing.assert_array_equal(po, o[a:b])
        np.testing.assert_array_equal(pf[0], fin[n])


def test_prefill_split_with_state_handoff():
    """prefill[0,T) vs prefill[0,100) -> state -> prefill[100,T) (T1 not a multiple of 64)."""
    rng = np.random.default_rng(45)
    T, T1 = 300, 100
    s = sequence_inputs(rng, [T], 2, 6, 128, dtype="bf16", init="normal")
    ro, rf = oracle_prefill(s)
    cut = lambda a, b, s0: dict(s, q=s["q"][a:b], k=s["k"][a:b], v=s["v"][a:b], g=s["g"][a:b],
                                beta=s["beta"][a:b], cu_seqlens=np.array([0, b - a], np.int32), initial_state=s0)
    o1, f1 = run_prefill(cut(0, T1, s["initial_state"]))
    o2, f2 = run_prefill(cut(T1, T, f1))
    assert rel_l2(np.concatenate([o1, o2]), ro) <= 2e-3
    assert rel_l2(f2, rf) <= 2e-3


@pytest.mark.parametrize("dtype,tol", [("bf16", 2e-3), ("f32", 1e-5)])
def test_chunked_equals_stepwise_on_gpu(dtype, tol):
    """The pages' two paths for one layer: GPU prefill vs GPU decode iterated token by token."""
    rng = np.random.default_rng(46)
    T = 150
    s = sequence_inputs(rng, [T], 2, 6, 128, dtype=dtype, init="normal")
    o, fin = run_prefill(s)
    st = _t(s["initial_state"])
    outs = []
    for t in range(T):
        ot = gdn.decode_step(_t(s["q"][t:t + 1]), _t(s["k"][t:t + 1]), _t(s["v"][t:t + 1]),
                             _t(s["g"][t:t + 1]), _t(s["beta"][t:t + 1]), st, o_dtype=torch.float32)
        outs.append(host(ot)[0])
    torch.cuda.synchronize()
    assert rel_l2(o, np.stack(outs)) <= tol
    assert rel_l2(fin[0], host(st)[0]) <= tol


# ------------------------------------------------------------------ degenerate cases

def _custom(rng, T, hk=1, hv=3, beta=None, g=None, unit_exact=False, init="normal"):
    s = sequence_inputs(rng, [T], hk, hv, 128, dtype="bf16", init=init)
    if beta is not None:
        s["beta"][:] = beta
    if g is not None:
        s["g"][:] = g
    return s


def test_beta_zero_pure_decay():
    s = _custom(np.random.default_rng(51), 130, beta=0.0)
    o, fin = run_prefill(s)
    ro, rf = oracle_prefill(s)
    assert rel_l2(o, ro) <= 2e-3 and rel_l2(fin, rf) <= 2e-3


def test_beta_one_overwrite_retrieves_values():
    """beta = 1, q = k (unit norm): o_t = v_t for any decay and history."""
    rng = np.random.default_rng(52)
    s = _custom(rng, 130, beta=1.0)
    s["q"] = s["k"].copy()
    o, _ = run_prefill(s)
    ro, _ = oracle_prefill(s)
    assert rel_l2(o, ro) <= 2e-3
    assert rel_l2(o, oracle.as_f64(s["v"])) <= 2e-2  # keys are unit only to bf16 precision


def test_no_decay_and_strong_decay():
    for g in (0.0, -30.0):
        s = _custom(np.random.default_rng(53), 140, g=g)
        o, fin = run_prefill(s)
        ro, rf = oracle_prefill(s)
        assert rel_l2(o, ro) <= 2e-3 and rel_l2(fin, rf) <= 2e-3, g


def test_slow_decay_long_sequence():
    """g scaled by 0.001 over T = 4096: the fp32 state must not drift."""
    rng = np.random.default_rng(54)
    s = sequence_inputs(rng, [4096], 1, 3, 128, dtype="bf16", init="normal", g_scale=0.001)
    o, fin = run_prefill(s)
    ro, rf = oracle_prefill(s)
    eo, ef = rel_l2(o, ro), rel_l2(fin, rf)
    print(f"slow decay rel-L2 o={eo:.3e} state={ef:.3e}")
    assert eo <= 2e-3 and ef <= 2e-3


def test_nan_in_one_head_does_not_leak():
    rng = np.random.default_rng(55)
    s = sequence_inputs(rng, [100, 80], 2, 6, 128, dtype="bf16", init="normal")
    s["v"][10, 4, 7] = 0x7FC0  # NaN in value head 4 of sequence 0
    o, fin = run_prefill(s)
    assert np.isnan(o[10:100, 4]).any()
    clean = np.ones(6, bool)
    clean[4] = False
    assert np.isfinite(o[:, clean]).all() and np.isfinite(o[100:]).all()
    assert np.isfinite(fin[1]).all() and np.isfinite(fin[0][clean]).all()
