"""GPU parity on seeded random shapes: the whole-layer prefill and the plain chunked prefill over
random packed batches (empty, one-token, chunk-boundary and multi-chunk sequences; 1, 2 or 4 key
heads with 1 to 6 value heads each; with and without conv history and initial states), each
followed by decode steps from its final states, all against the fp64 oracle.

Gates as in the fixed-shape tests: rel-L2 2e-3 for every output from bf16 inputs (y, o, final
states, also over each sequence's first 128 tokens), exact conv history, 1e-5 for the fp32
decode steps after the prefill.
"""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits
from tests.helpers import dev, host, rel_l2, as_f64

torch = pytest.importorskip("torch")
import gated_delta_rule_35_amd as gdn  # noqa: E402

pytestmark = pytest.mark.gpu

D = 128
LEN_POOL = [0, 1, 2, 3, 5, 63, 64, 65, 127, 128, 129, 200, 257, 511]


def _shape(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 5))
    lens = [int(r.choice(LEN_POOL)) for _ in range(n)]
    if seed % 3 == 0:  # one long sequence: long enough for the two-stage launch
        lens[int(r.integers(0, n))] = int(r.integers(600, 1400))
    hk = int(r.choice([1, 2, 4]))
    grp = int(r.choice([1, 2, 3, 4, 6] if hk < 4 else [1, 2, 3]))
    return dict(lens=lens, hk=hk, hv=hk * grp, hist=bool(r.integers(0, 2)), init=bool(r.integers(0, 2)),
                z_pad=int(r.choice([0, 8, 64])), scale=float(r.choice([1.0, 0.5])))


SEEDS = list(range(7000, 7040))


def _case(rng, sh):
    lens, hk, hv = sh["lens"], sh["hk"], sh["hv"]
    T = int(sum(lens))
    C = (2 * hk + hv) * D
    f = np.float32
    return dict(
        x=f32_to_bf16_bits(rng.standard_normal((T, C)).astype(f) * f(1.43)),
        w=f32_to_bf16_bits(rng.uniform(-0.5, 0.5, (C, 4)).astype(f)),
        cs=f32_to_bf16_bits(rng.standard_normal((len(lens), C, 3)).astype(f) * f(1.43)) if sh["hist"] else None,
        g=(-0.05 * np.logaddexp(0, rng.standard_normal((T, hv)))).astype(f),
        beta=(1 / (1 + np.exp(-rng.standard_normal((T, hv))))).astype(f),
        s0=(rng.standard_normal((len(lens), hv, D, D)) * 0.01).astype(f) if sh["init"] else None,
        z=f32_to_bf16_bits(rng.standard_normal((T, hv, D)).astype(f)),
        nw=f32_to_bf16_bits((1 + 0.1 * rng.standard_normal(D)).astype(f)),
        cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
    )


def _first128(a, ref, cu):
    rows = np.concatenate([np.arange(s, min(e, s + 128)) for s, e in zip(cu[:-1], cu[1:])] + [np.arange(0)])
    return rel_l2(a[rows], ref[rows]) if len(rows) else 0.0


@pytest.mark.parametrize("seed", SEEDS)
def test_layer_prefill_then_decode_random_shape(seed):
    sh = _shape(seed)
    rng = np.random.default_rng(seed + 100)
    d = _case(rng, sh)
    T, hv, hk = int(d["cu"][-1]), sh["hv"], sh["hk"]
    print(f"seed {seed}: {sh}", flush=True)
    # whole layer in one call
    cs = None if d["cs"] is None else dev(d["cs"])
    if sh["z_pad"]:
        zb = torch.zeros((T, hv * D + sh["z_pad"]), dtype=torch.bfloat16, device="cuda")
        zb[:, :hv * D] = dev(d["z"]).view(T, hv * D)
        z = zb[:, :hv * D].view(T, hv, D)
    else:
        z = dev(d["z"])
    o = torch.empty((T, hv, D), dtype=torch.float32, device="cuda")
    y, fin = gdn.layer_prefill(dev(d["x"]), dev(d["w"]), dev(d["g"]), dev(d["beta"]), dev(d["cu"]), z, dev(d["nw"]),
                               num_k_heads=hk, conv_state=cs, scale=sh["scale"],
                               initial_state=None if d["s0"] is None else dev(d["s0"]), o=o, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rcs, rfin = oracle.prefill_conv_recurrence(d["x"], d["w"], d["cu"], d["cs"], d["g"], d["beta"], d["s0"],
                                                   hk, hv, scale=sh["scale"])
    ry = oracle.gated_rmsnorm(ro, d["z"], d["nw"])
    y, o, fin = host(y), host(o), host(fin)
    if T:
        assert rel_l2(y, ry) <= 2e-3 and rel_l2(o, ro) <= 2e-3
        assert _first128(y, ry, d["cu"]) <= 2e-3 and _first128(o, ro, d["cu"]) <= 2e-3
    assert rel_l2(fin, rfin) <= 2e-3
    if cs is not None:
        np.testing.assert_array_equal(as_f64(host(cs)), rcs)
    # two decode steps of every sequence from the final states (fp32 inputs, fp32 path)
    st = torch.from_numpy(fin).cuda()
    rst = fin.astype(np.float64)
    for step in range(2):
        r = np.random.default_rng(seed * 10 + step)
        B = len(sh["lens"])
        q = (r.standard_normal((B, hk, D)) / np.sqrt(D)).astype(np.float32)
        k = r.standard_normal((B, hk, D)).astype(np.float32)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = r.standard_normal((B, hv, D)).astype(np.float32)
        g = (-0.05 * np.logaddexp(0, r.standard_normal((B, hv)))).astype(np.float32)
        b = (1 / (1 + np.exp(-r.standard_normal((B, hv))))).astype(np.float32)
        od = gdn.decode_step(dev(q), dev(k), dev(v), dev(g), dev(b), st, o_dtype=torch.float32, scale=sh["scale"])
        rod, rst = oracle.decode_step(q, k, v, g, b, rst, scale=sh["scale"])
        torch.cuda.synchronize()
        assert rel_l2(host(od), rod) <= 1e-5 and rel_l2(host(st), rst) <= 1e-5, step


@pytest.mark.parametrize("seed", SEEDS[::2])
def test_chunked_prefill_random_shape(seed):
    """The plain call on the conv outputs (bf16 q, k, v as separate arrays) of the same shapes."""
    sh = _shape(seed)
    rng = np.random.default_rng(seed + 200)
    lens, hk, hv = sh["lens"], sh["hk"], sh["hv"]
    T = int(sum(lens))
    print(f"seed {seed}: {sh}", flush=True)
    f = np.float32
    q = rng.standard_normal((T, hk, D)).astype(f)
    k = rng.standard_normal((T, hk, D)).astype(f)
    q /= np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-6)
    k /= np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-6)
    q, k = f32_to_bf16_bits(q), f32_to_bf16_bits(k)
    v = f32_to_bf16_bits(rng.standard_normal((T, hv, D)).astype(f))
    g = (-0.05 * np.logaddexp(0, rng.standard_normal((T, hv)))).astype(f)
    beta = (1 / (1 + np.exp(-rng.standard_normal((T, hv))))).astype(f)
    s0 = (rng.standard_normal((len(lens), hv, D, D)) * 0.01).astype(f) if sh["init"] else None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, fin = gdn.prefill_chunked(dev(q), dev(k), dev(v), dev(g), dev(beta), dev(cu), scale=sh["scale"],
                                 initial_state=None if s0 is None else dev(s0), o_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rfin = oracle.recurrence(q, k, v, g, beta, cu, s0, scale=sh["scale"])
    o, fin = host(o), host(fin)
    if T:
        assert rel_l2(o, ro) <= 2e-3 and _first128(o, ro, cu) <= 2e-3
    assert rel_l2(fin, rfin) <= 2e-3
