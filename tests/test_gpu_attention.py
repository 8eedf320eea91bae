"""GPU parity of agnes_attn_prefill (the global attention layer) against the fp64 oracle.

Tolerances (derived from the arithmetic): the products take bf16 operands — q after norm and
rotary, k as stored in k_out, v, and the softmax weights — each rounded once to 8 significant
bits (relative 2^-9), with fp32 accumulation and fp32 softmax statistics.  A score or an output
element then carries at most about 2 x 2^-9 = 3.9e-3 relative error, so the fp32 o is gated at
rel-L2 4e-3, on the whole tensor and on each sequence's first 64 rows.  The bf16 o of the same
call is the round-to-nearest-even of the fp32 o, bit for bit (same kernel, other store).  k_out
is within one bf16 ulp of RNE(oracle) everywhere and bit-exact for >= 99 % of its elements (the
fp32 norm and rotary may round differently near a tie); v_out is an exact copy.
"""
import numpy as np
import pytest

import oracle
from synth import attn_prefill_inputs, attn_decode_inputs, f32_to_bf16_bits
from tests.helpers import dev, host, rel_l2, as_f64, check_bf16_out

torch = pytest.importorskip("torch")
import gated_delta_rule_35_amd as gdn  # noqa: E402

pytestmark = pytest.mark.gpu

D = 256
TOL = 4e-3


def _run(d, o_dtype=torch.float32, positions=None, v_out=False):
    T, hkv = d["k"].shape[0], d["k"].shape[1]
    vo = torch.empty((T, hkv, D), dtype=torch.bfloat16, device="cuda") if v_out else None
    o, ko = gdn.attn_prefill(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["gate"]), dev(d["qw"]), dev(d["kw"]),
                             dev(d["cu"]), positions=None if positions is None else dev(positions), v_out=vo,
                             o_dtype=o_dtype)
    torch.cuda.synchronize()
    return host(o), host(ko), (None if vo is None else host(vo))


def _first64(o, ro, cu):
    rows = np.concatenate([np.arange(a, min(b, a + 64)) for a, b in zip(cu[:-1], cu[1:])])
    return rel_l2(o[rows], ro[rows])


@pytest.mark.parametrize("hq,hkv", [(6, 1), (24, 4)])
def test_attn_prefill_varlen(hq, hkv):
    """Ragged batch: sequences of 1 and 2 tokens, an empty one, exact and partial 64-key blocks
    and 128-query blocks, several blocks."""
    rng = np.random.default_rng(500 + hq)
    lens = [70, 1, 0, 131, 64, 2, 200, 129]
    d = attn_prefill_inputs(rng, lens, hq, hkv)
    o, ko, vo = _run(d, v_out=True)
    ro, rk = oracle.attention_prefill(d["q"], d["k"], d["v"], d["gate"], d["cu"], d["qw"], d["kw"])
    e, e64 = rel_l2(o, ro), _first64(o, ro, d["cu"])
    print(f"attention prefill Hq={hq}: o rel-L2 {e:.3e}, first-64 {e64:.3e}")
    assert e <= TOL and e64 <= TOL
    exact = check_bf16_out(ko, rk, exact_frac=0.99)
    print(f"k_out bit-exact fraction {exact:.5f}")
    np.testing.assert_array_equal(vo, d["v"])


def test_attn_prefill_bf16_output_is_rne_of_fp32_output():
    rng = np.random.default_rng(510)
    d = attn_prefill_inputs(rng, [150, 37], 6, 1)
    o32, k32, _ = _run(d)
    o16, k16, _ = _run(d, torch.bfloat16)
    np.testing.assert_array_equal(o16, f32_to_bf16_bits(o32))
    np.testing.assert_array_equal(k16, k32)


def test_attn_prefill_three_axis_positions():
    """Explicit (text, height, width) positions that differ per axis (image-like tokens): the
    rotary follows axis j mod 3 for frequency j."""
    rng = np.random.default_rng(520)
    lens = [96, 40]
    d = attn_prefill_inputs(rng, lens, 6, 1)
    T = sum(lens)
    pos = rng.integers(0, 5000, size=(3, T)).astype(np.int32)
    o, ko, _ = _run(d, positions=pos)
    ro, rk = oracle.attention_prefill(d["q"], d["k"], d["v"], d["gate"], d["cu"], d["qw"], d["kw"], pos3=pos)
    e = rel_l2(o, ro)
    print(f"attention prefill, three-axis positions: o rel-L2 {e:.3e}")
    assert e <= TOL
    check_bf16_out(ko, rk, exact_frac=0.99)


def test_attn_prefill_t8192_sampled_rows():
    """The bench workload (T = 8192, one sequence, 24 query / 4 KV heads); the oracle follows
    rows at block edges and the end, for query heads at the edges of their KV groups."""
    rng = np.random.default_rng(530)
    T, hq, hkv = 8192, 24, 4
    d = attn_prefill_inputs(rng, [T], hq, hkv)
    o, ko, _ = _run(d)
    rows = [0, 1, 63, 64, 127, 128, 1000, 4095, 4096, 8190, 8191]
    heads = [0, 5, 6, 17, 23]
    pos = oracle.text_positions(d["cu"], T)
    ang = oracle.rope_angles(pos)
    kr = oracle.apply_rotary(oracle.rms_norm_heads(d["k"], d["kw"]), ang)
    qr = np.zeros((T, hq, D))
    qr[rows] = oracle.apply_rotary(oracle.rms_norm_heads(d["q"][rows], d["qw"]), ang[rows])
    ro = oracle.causal_attention_rows(qr, kr, d["v"], d["cu"], rows, heads)
    ro = ro * (1.0 / (1.0 + np.exp(-as_f64(d["gate"])[rows][:, heads])))
    e = rel_l2(o[rows][:, heads], ro)
    print(f"attention prefill T=8192 sampled rows: o rel-L2 {e:.3e}")
    assert e <= TOL
    check_bf16_out(ko, kr, exact_frac=0.99)


# ---------------------------------------------------------------- decode

def _decode(d, o_dtype=torch.float32, lens=None):
    kc, vc = dev(d["k_cache"]), dev(d["v_cache"])
    lens = d["lens"] if lens is None else lens
    o = gdn.attn_decode(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["gate"]), dev(d["qw"]), dev(d["kw"]), kc, vc,
                        dev(np.asarray(lens, np.int32)), o_dtype=o_dtype)
    torch.cuda.synchronize()
    return host(o), host(kc), host(vc)


def _decode_check(d, lens, lmax):
    o, kc, vc = _decode(d, lens=lens)
    live = [b for b in range(len(lens)) if 0 <= lens[b] < lmax]
    ro, rkc, rvc = oracle.attention_decode(d["q"][live], d["k"][live], d["v"][live], d["gate"][live],
                                           d["k_cache"][live], d["v_cache"][live], np.asarray(lens)[live],
                                           d["qw"], d["kw"])
    e = rel_l2(o[live], ro)
    for b in range(len(lens)):
        if b not in live:  # padding: zero output, cache untouched
            assert not o[b].any()
            np.testing.assert_array_equal(kc[b], d["k_cache"][b])
            np.testing.assert_array_equal(vc[b], d["v_cache"][b])
    for i, b in enumerate(live):
        L = lens[b]
        others = np.ones(lmax, bool)
        others[L] = False
        np.testing.assert_array_equal(kc[b][others], d["k_cache"][b][others])
        np.testing.assert_array_equal(vc[b][others], d["v_cache"][b][others])
        np.testing.assert_array_equal(vc[b][L], d["v"][b])
        check_bf16_out(kc[b][L], rkc[i][L], exact_frac=0.99)
    return e


def test_attn_decode_mixed_lengths_and_padding():
    """Empty cache, one token, a 64-key block edge, a long entry, and a padding entry (length
    outside the cache)."""
    rng = np.random.default_rng(540)
    lmax = 800
    lens = [0, 1, 63, 64, 700, 800]
    d = attn_decode_inputs(rng, [min(x, lmax) for x in lens], lmax)
    e = _decode_check(d, lens, lmax)
    print(f"attention decode mixed lengths: o rel-L2 {e:.3e}")
    assert e <= TOL


def test_attn_decode_long_context_splits():
    """Caches of 8191 and 5000 tokens: the keys are split over several workgroups and merged."""
    rng = np.random.default_rng(550)
    lmax = 8192
    lens = [8191, 5000]
    d = attn_decode_inputs(rng, lens, lmax)
    e = _decode_check(d, lens, lmax)
    print(f"attention decode long context: o rel-L2 {e:.3e}")
    assert e <= TOL


def test_attn_decode_bf16_output_is_rne_of_fp32_output():
    rng = np.random.default_rng(560)
    d = attn_decode_inputs(rng, [10, 300], 512)
    o32, _, _ = _decode(d)
    o16, _, _ = _decode(d, torch.bfloat16)
    np.testing.assert_array_equal(o16, f32_to_bf16_bits(o32))


def test_attn_decode_continues_prefill():
    """A GPU prefill of 100 tokens fills the cache (its k_out and v_out are the cache rows), then
    three decode steps follow: their outputs are the oracle prefill's rows 100..102."""
    rng = np.random.default_rng(570)
    T, lmax, hq, hkv = 103, 128, 24, 4
    d = attn_prefill_inputs(rng, [T], hq, hkv)
    kc = torch.zeros((1, lmax, hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((1, lmax, hkv, D), dtype=torch.bfloat16, device="cuda")
    cu = np.array([0, 100], np.int32)
    gdn.attn_prefill(dev(d["q"][:100]), dev(d["k"][:100]), dev(d["v"][:100]), dev(d["gate"][:100]), dev(d["qw"]),
                     dev(d["kw"]), dev(cu), k_out=kc[0, :100], v_out=vc[0, :100])
    outs = []
    for t in range(100, T):
        o = gdn.attn_decode(dev(d["q"][t:t + 1]), dev(d["k"][t:t + 1]), dev(d["v"][t:t + 1]), dev(d["gate"][t:t + 1]),
                            dev(d["qw"]), dev(d["kw"]), kc, vc, dev(np.array([t], np.int32)), o_dtype=torch.float32)
        outs.append(host(o)[0])
    torch.cuda.synchronize()
    ro, _ = oracle.attention_prefill(d["q"], d["k"], d["v"], d["gate"], [0, T], d["qw"], d["kw"])
    e = rel_l2(np.stack(outs), ro[100:])
    print(f"attention decode after prefill: o rel-L2 {e:.3e}")
    assert e <= TOL
