"""C-ABI boundary on the CPU: the library loads, exports exactly the header's functions, and
every argument check returns its documented status before anything is launched.

Pointer values below are never dereferenced: every call is built to fail a host-side check.
"""
import ctypes
import os
import re
import subprocess

import pytest

from gated_delta_rule_35_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "agnes_gdn.h")

INV, UNS, WS = _lib.ERR_INVALID_ARG, _lib.ERR_UNSUPPORTED, _lib.ERR_WORKSPACE
BF16, F32 = _lib.BF16, _lib.F32
P = [0x10000000 * (i + 1) for i in range(12)]  # distinct, 16-byte aligned fake device pointers


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from gated_delta_rule_35_amd.build import build
        build()
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(agnes_\w+)\s*\(", text, re.M)))


def test_header_declares_the_layer_calls():
    names = header_functions()
    for n in ("agnes_gdn_conv", "agnes_gdn_prefill_chunked", "agnes_gdn_decode_step",
              "agnes_gdn_gated_rmsnorm", "agnes_attn_prefill", "agnes_attn_decode"):
        assert n in names
    assert set(names) == set(_lib.SIGNATURES)


def test_library_exports_exactly_the_header(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r"\b(agnes_\w+)\b", out)))
    assert exported == header_functions()


def test_status_strings_and_version(lib):
    assert lib.agnes_gdn_version().decode().count(".") == 2
    for s in (0, -1, -2, -3, -4):
        assert lib.agnes_gdn_status_string(s)
    assert lib.agnes_gdn_last_hip_error() == 0


def conv(lib, **kw):
    a = dict(x=P[0], xs=512, y=P[1], ys=512, dt=BF16, w=P[2], b=None, cu=P[3], n=2, T=10, C=512, K=4,
             st=None, l2=2, hd=128, eps=1e-6)
    a.update(kw)
    return lib.agnes_gdn_conv(a["x"], a["xs"], a["y"], a["ys"], a["dt"], a["w"], a["b"], a["cu"], a["n"], a["T"],
                              a["C"], a["K"], a["st"], a["l2"], a["hd"], a["eps"], None)


def test_conv_checks(lib):
    assert conv(lib, x=None) == INV
    assert conv(lib, dt=7) == INV
    assert conv(lib, x=P[0] + 8) == INV                 # misaligned
    assert conv(lib, C=500, xs=500, ys=500) == INV      # channels % 8
    assert conv(lib, xs=256) == INV                     # stride < channels
    assert conv(lib, K=3) == UNS
    assert conv(lib, hd=64) == UNS                      # L2 step needs 128-channel heads
    assert conv(lib, l2=5) == INV                       # 5 * 128 > 512 channels
    assert conv(lib, eps=float("nan")) == INV
    assert conv(lib, cu=None, n=10, T=10) == INV        # decode mode needs conv_state
    assert conv(lib, cu=None, n=4, T=10, st=P[4]) == INV  # decode: one token per sequence
    assert conv(lib, n=0, T=10) == INV
    assert conv(lib, y=P[0] + 512) == INV               # y overlaps x
    assert lib.agnes_gdn_last_hip_error() == 0


def prefill(lib, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], dt=BF16, qs=2 * 128, vs=6 * 128, g=P[3], b=P[4], cu=P[5], n=1, T=64,
             hk=2, hv=6, hd=128, sc=1.0, s0=P[6], s1=P[7], o=P[8], odt=F32, ws=None, wsb=0)
    a.update(kw)
    return lib.agnes_gdn_prefill_chunked(a["q"], a["k"], a["v"], a["dt"], a["qs"], a["vs"], a["g"], a["b"],
                                         a["cu"], a["n"], a["T"], a["hk"], a["hv"], a["hd"], a["sc"], a["s0"],
                                         a["s1"], a["o"], a["odt"], a["ws"], a["wsb"], None)


def test_prefill_checks(lib):
    assert prefill(lib, hd=64) == UNS
    assert prefill(lib, hv=5) == UNS                    # Hv % Hk
    assert prefill(lib, q=None) == INV
    assert prefill(lib, cu=None) == INV
    assert prefill(lib, q=P[0] + 2) == INV              # misaligned
    assert prefill(lib, qs=100) == INV                  # stride < Hk * 128
    assert prefill(lib, qs=2 * 128 + 4) == INV          # stride % 8
    assert prefill(lib, n=0) == INV                     # tokens without sequences
    assert prefill(lib, n=-1) == INV
    assert prefill(lib, s1=P[6] + 1024) == INV          # partial overlap of the two states
    assert prefill(lib, o=P[0] + 64) == INV             # o overlaps q
    assert prefill(lib, sc=float("inf")) == INV
    assert prefill(lib, odt=3) == INV
    # bf16 inputs need a workspace: missing, too small or misaligned -> AGNES_ERR_WORKSPACE
    need = lib.agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 128, BF16)
    assert need > 0 and need % 256 == 0
    assert prefill(lib) == WS
    assert prefill(lib, ws=P[9], wsb=need - 1) == WS
    assert prefill(lib, ws=P[9] + 16, wsb=need) == WS
    assert lib.agnes_gdn_prefill_workspace_size(3, 1000, 2, 6, 128, BF16) > need
    assert lib.agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 128, F32) == 0
    assert lib.agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 64, BF16) == 0
    assert lib.agnes_gdn_prefill_workspace_size(1, 64, 2, 5, 128, BF16) == 0


def decode(lib, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], dt=BF16, qs=2 * 128, vs=6 * 128, g=P[3], b=P[4], B=4, hk=2, hv=6, hd=128,
             sc=1.0, st=P[5], o=P[6], odt=F32)
    a.update(kw)
    return lib.agnes_gdn_decode_step(a["q"], a["k"], a["v"], a["dt"], a["qs"], a["vs"], a["g"], a["b"], a["B"],
                                     a["hk"], a["hv"], a["hd"], a["sc"], a["st"], a["o"], a["odt"], None)


def test_decode_checks(lib):
    assert decode(lib, hd=96) == UNS
    assert decode(lib, hv=7) == UNS
    assert decode(lib, st=None) == INV
    assert decode(lib, st=P[5] + 4) == INV              # state must be 16-byte aligned
    assert decode(lib, o=P[5] + 4096) == INV            # o inside the state
    assert decode(lib, B=-1) == INV
    assert decode(lib, vs=100) == INV


def norm(lib, **kw):
    a = dict(o=P[0], odt=BF16, z=P[1], w=P[2], zdt=BF16, eps=1e-6, rows=100, dim=128, y=P[3], ydt=BF16)
    a.update(kw)
    return lib.agnes_gdn_gated_rmsnorm(a["o"], a["odt"], a["z"], a["w"], a["zdt"], a["eps"], a["rows"], a["dim"],
                                       a["y"], a["ydt"], None)


def test_norm_checks(lib):
    assert norm(lib, dim=64) == UNS
    assert norm(lib, rows=-1) == INV
    assert norm(lib, o=None) == INV
    assert norm(lib, y=P[0] + 256) == INV               # partial overlap of o and y
    assert norm(lib, y=P[0], ydt=F32) == INV            # aliasing needs equal dtypes
    assert norm(lib, y=P[1] + 16) == INV                # y overlaps z
    assert norm(lib, eps=-1.0) == INV


def fused(lib, **kw):
    a = dict(x=P[0], xs=10 * 128, dt=BF16, w=P[1], b=None, cs=P[2], g=P[3], be=P[4], z=P[5], nw=P[6], st=P[7],
             sl=None, S=4, B=4, hk=2, hv=6, hd=128, sc=1.0, e1=1e-6, e2=1e-6, y=P[8], o=None, odt=BF16)
    a.update(kw)
    return lib.agnes_gdn_decode_fused(a["x"], a["xs"], a["dt"], a["w"], a["b"], a["cs"], a["g"], a["be"], a["z"],
                                      a["nw"], a["st"], a["sl"], a["S"], a["B"], a["hk"], a["hv"], a["hd"], a["sc"],
                                      a["e1"], a["e2"], a["y"], a["o"], a["odt"], None)


def test_decode_fused_checks(lib):
    assert fused(lib, B=0, x=None, y=None) == 0         # empty batch: nothing to do
    assert fused(lib, hd=64) == UNS
    assert fused(lib, hv=7) == UNS                      # Hv % Hk
    assert fused(lib, x=None) == INV
    assert fused(lib, cs=None) == INV
    assert fused(lib, S=3) == INV                       # no slot array: a slot per entry needed
    assert fused(lib, xs=10 * 128 - 8) == INV           # row stride below the channel count
    assert fused(lib, xs=10 * 128 + 4) == INV           # row stride % 8
    assert fused(lib, x=P[0] + 8) == INV                # misaligned
    assert fused(lib, st=P[7] + 4) == INV
    assert fused(lib, dt=5) == INV
    assert fused(lib, e2=float("nan")) == INV
    assert fused(lib, sc=float("inf")) == INV
    assert fused(lib, B=-1) == INV
    assert fused(lib, y=P[7] + 4096) == INV             # y inside the state pool
    assert fused(lib, o=P[8] + 256) == INV              # o overlaps y
    assert fused(lib, cs=P[0] + 1024) == INV            # conv history overlaps x
    assert fused(lib, y=P[5] + 64) == INV               # y overlaps z
    assert lib.agnes_gdn_last_hip_error() == 0


def pfused(lib, **kw):
    a = dict(x=P[0], xs=10 * 128, dt=BF16, w=P[1], b=None, cs=None, g=P[3], be=P[4], cu=P[5], n=1, T=64, hk=2, hv=6,
             hd=128, sc=1.0, eps=1e-6, s0=None, s1=P[7], o=P[8], odt=F32, ws=None, wsb=0)
    a.update(kw)
    return lib.agnes_gdn_prefill_fused(a["x"], a["xs"], a["dt"], a["w"], a["b"], a["cs"], a["g"], a["be"], a["cu"],
                                       a["n"], a["T"], a["hk"], a["hv"], a["hd"], a["sc"], a["eps"], a["s0"], a["s1"],
                                       a["o"], a["odt"], a["ws"], a["wsb"], None)


def test_prefill_fused_checks(lib):
    assert pfused(lib, dt=F32) == UNS                   # the fused path takes bf16 x only
    assert pfused(lib, hd=64) == UNS
    assert pfused(lib, hv=5, xs=9 * 128) == UNS         # Hv % Hk
    assert pfused(lib, w=None) == INV
    assert pfused(lib, x=None) == INV
    assert pfused(lib, xs=10 * 128 - 8) == INV          # stride below the channel count
    assert pfused(lib, x=P[0] + 8) == INV
    assert pfused(lib, eps=-1.0) == INV
    assert pfused(lib, o=P[0] + 64) == INV              # o overlaps x
    assert pfused(lib, cs=P[0] + 128) == INV            # conv history overlaps x
    assert pfused(lib, n=0) == INV                      # tokens without sequences
    need = lib.agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 128, BF16)
    assert pfused(lib) == WS
    assert pfused(lib, ws=P[9], wsb=need - 1) == WS
    assert lib.agnes_gdn_last_hip_error() == 0


def layer(lib, **kw):
    a = dict(x=P[0], xs=10 * 128, dt=BF16, w=P[1], b=None, cs=None, g=P[3], be=P[4], cu=P[5], n=1, T=64, hk=2, hv=6,
             hd=128, sc=1.0, eps=1e-6, s0=None, s1=P[7], z=P[2], zs=6 * 128, nw=P[6], neps=1e-6, y=P[8], o=None,
             odt=BF16, ws=None, wsb=0)
    a.update(kw)
    return lib.agnes_gdn_layer_prefill(a["x"], a["xs"], a["dt"], a["w"], a["b"], a["cs"], a["g"], a["be"], a["cu"],
                                       a["n"], a["T"], a["hk"], a["hv"], a["hd"], a["sc"], a["eps"], a["s0"], a["s1"],
                                       a["z"], a["zs"], a["nw"], a["neps"], a["y"], a["o"], a["odt"], a["ws"],
                                       a["wsb"], None)


def test_layer_prefill_checks(lib):
    assert layer(lib, dt=F32) == UNS                    # bf16 x only
    assert layer(lib, hd=64) == UNS
    assert layer(lib, z=None) == INV
    assert layer(lib, y=None) == INV
    assert layer(lib, nw=None) == INV
    assert layer(lib, zs=6 * 128 - 8) == INV            # z stride below a token's heads
    assert layer(lib, zs=6 * 128 + 4) == INV            # z rows must stay 16-byte aligned
    assert layer(lib, neps=-1.0) == INV
    assert layer(lib, neps=float("nan")) == INV
    assert layer(lib, y=P[2] + 256) == INV              # y overlaps z
    assert layer(lib, o=P[8] + 512) == INV              # o overlaps y
    assert layer(lib, y=P[0] + 64) == INV               # y overlaps x
    assert layer(lib, n=0) == INV
    need = lib.agnes_gdn_layer_prefill_workspace_size(1, 64, 2, 6, 128)
    assert need >= lib.agnes_gdn_prefill_workspace_size(1, 64, 2, 6, 128, BF16)
    assert layer(lib) == WS
    assert layer(lib, ws=P[9], wsb=need - 1) == WS
    assert lib.agnes_gdn_layer_prefill_workspace_size(1, 64, 2, 5, 128) == 0
    assert lib.agnes_gdn_last_hip_error() == 0


def attn(lib, **kw):
    T, hq, hkv = 100, 24, 4
    a = dict(q=P[0], qs=hq * 256, k=P[1], ks=hkv * 256, v=P[2], vs=hkv * 256, g=P[3], gs=hq * 256, qw=P[4], kw=P[4] + 512,
             pos=None, ps=0, cu=P[5], n=1, T=T, hq=hq, hkv=hkv, hd=256, rd=64, base=1e7, eps=1e-6, sc=0.0, ko=P[6],
             kos=hkv * 256, vo=None, vos=0, o=P[7], odt=BF16, ws=None, wsb=0)
    a.update(kw)
    return lib.agnes_attn_prefill(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"], a["gs"], a["qw"], a["kw"],
                                  a["pos"], a["ps"], a["cu"], a["n"], a["T"], a["hq"], a["hkv"], a["hd"], a["rd"],
                                  a["base"], a["eps"], a["sc"], a["ko"], a["kos"], a["vo"], a["vos"], a["o"], a["odt"],
                                  a["ws"], a["wsb"], None)


def test_attn_prefill_checks(lib):
    assert attn(lib, n=0, T=0, q=None, k=None, v=None, g=None, ko=None, o=None) == 0  # empty batch
    assert attn(lib, hd=128) == UNS
    assert attn(lib, rd=32) == UNS
    assert attn(lib, hq=10) == UNS                      # Hq % Hkv
    assert attn(lib, ko=None) == INV                    # k_out is what the attention reads
    assert attn(lib, g=None) == INV
    assert attn(lib, qw=None) == INV
    assert attn(lib, qs=24 * 256 - 8) == INV            # stride below the heads
    assert attn(lib, ks=4 * 256 + 4) == INV             # stride % 8
    assert attn(lib, q=P[0] + 8) == INV                 # misaligned
    assert attn(lib, qw=P[4] + 2) == INV
    assert attn(lib, pos=P[8], ps=99) == INV            # positions stride below T
    assert attn(lib, base=0.0) == INV
    assert attn(lib, eps=float("nan")) == INV
    assert attn(lib, odt=5) == INV
    assert attn(lib, n=0) == INV                        # tokens without sequences
    assert attn(lib, o=P[0] + 512) == INV               # o overlaps q
    assert attn(lib, ko=P[1]) == INV                    # k_out overlaps k
    assert attn(lib, vo=P[7] + 1024, vos=1024) == INV   # v_out overlaps o
    need = lib.agnes_attn_prefill_workspace_size(1, 100)
    assert need > 0
    assert attn(lib) == WS
    assert attn(lib, ws=P[9], wsb=need - 1) == WS
    assert attn(lib, ws=P[9] + 16, wsb=need) == WS      # not 256-byte aligned
    assert lib.agnes_gdn_last_hip_error() == 0


def adec(lib, **kw):
    B, hq, hkv, L = 8, 24, 4, 1000
    a = dict(q=P[0], qs=hq * 256, k=P[1], ks=hkv * 256, v=P[2], vs=hkv * 256, g=P[3], gs=hq * 256, qw=P[4],
             kw=P[4] + 512, pos=None, ps=0, kc=P[5], vc=P[6], L=L, lens=P[7], B=B, hq=hq, hkv=hkv, hd=256, rd=64,
             base=1e7, eps=1e-6, sc=0.0, o=P[8], odt=BF16, ws=None, wsb=0)
    a.update(kw)
    return lib.agnes_attn_decode(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"], a["gs"], a["qw"], a["kw"],
                                 a["pos"], a["ps"], a["kc"], a["vc"], a["L"], a["lens"], a["B"], a["hq"], a["hkv"],
                                 a["hd"], a["rd"], a["base"], a["eps"], a["sc"], a["o"], a["odt"], a["ws"], a["wsb"],
                                 None)


def test_attn_decode_checks(lib):
    assert adec(lib, B=0, q=None, kc=None) == 0         # empty batch
    assert adec(lib, hd=128) == UNS
    assert adec(lib, hq=22) == UNS                      # Hq % Hkv
    assert adec(lib, L=0) == INV                        # no cache rows
    assert adec(lib, kc=None) == INV
    assert adec(lib, lens=None) == INV
    assert adec(lib, qs=24 * 256 - 8) == INV
    assert adec(lib, vs=4 * 256 + 4) == INV
    assert adec(lib, kc=P[5] + 8) == INV                # misaligned
    assert adec(lib, pos=P[9], ps=7) == INV             # positions stride below the batch
    assert adec(lib, sc=float("nan")) == INV
    assert adec(lib, vc=P[5] + 4096) == INV             # caches overlap
    assert adec(lib, o=P[0] + 1024) == INV              # o overlaps q
    need = lib.agnes_attn_decode_workspace_size(8, 24, 4, 1000)
    assert need > 0
    assert adec(lib) == WS
    assert adec(lib, ws=P[10], wsb=need - 1) == WS
    assert lib.agnes_gdn_last_hip_error() == 0


def test_status_and_measurement_calls_check_their_arguments(lib):
    """The status query, the wait-limit hook and the two measurement kernels reject bad
    arguments before touching the device."""
    import ctypes
    flags = ctypes.c_uint32(7)
    assert lib.agnes_gdn_workspace_status(None, ctypes.addressof(flags), None) == INV
    assert lib.agnes_gdn_workspace_status(P[0], None, None) == INV
    assert lib.agnes_gdn_workspace_status(P[0] + 2, ctypes.addressof(flags), None) == INV  # misaligned
    assert flags.value == 7
    assert lib.agnes_gdn_set_wait_limit(0) == 0
    assert lib.agnes_gdn_ceiling_rmw_stream(None, 1024, None) == INV
    assert lib.agnes_gdn_ceiling_rmw_stream(P[0], 1000, None) == INV                # not a multiple of 16
    assert lib.agnes_gdn_ceiling_rmw_stream(P[0] + 8, 1024, None) == INV            # misaligned
    assert lib.agnes_gdn_ceiling_mfma(None, 4, 4, None) == INV
    assert lib.agnes_gdn_ceiling_mfma(P[0], 0, 4, None) == INV
    assert lib.agnes_gdn_ceiling_mfma(P[0], 4, (1 << 20) + 1, None) == INV
    assert lib.agnes_gdn_last_hip_error() == 0



def test_stage_cuts_are_checked_on_the_host(lib):
    """The stage cuts must increase strictly inside (0, 40), at most 7 of them; any other list is
    refused and leaves the setting as it was (host-only, no device call)."""
    import ctypes

    def cuts(*v):
        return (ctypes.c_int32 * max(len(v), 1))(*v), len(v)

    for bad in [(0,), (40,), (24, 24), (30, 20), (-1,), tuple(range(1, 9))]:
        assert lib.agnes_gdn_set_prefill_stages(*cuts(*bad)) == INV, bad
    assert lib.agnes_gdn_set_prefill_stages(None, 1) == INV
    assert lib.agnes_gdn_set_prefill_stages(None, -2) == INV
    assert lib.agnes_gdn_set_prefill_stages(None, 0) == 0
    assert lib.agnes_gdn_set_prefill_stages(*cuts(1, 2, 3, 4, 5, 6, 39)) == 0
    assert lib.agnes_gdn_set_prefill_stages(*cuts(26)) == 0
    assert lib.agnes_gdn_set_prefill_stages(None, -1) == 0  # the defaults again
    assert lib.agnes_gdn_last_hip_error() == 0

def test_noalloc_refuses_a_workspace_beyond_its_own_on_the_host(lib):
    """The fixed-workspace call rejects a problem whose workspace exceeds its 64 MiB before any
    device call (the size query is host arithmetic)."""
    T = 8192
    assert lib.agnes_gdn_layer_prefill_workspace_size(1, T, 16, 48, 128) > (64 << 20)
    st = lib.agnes_gdn_layer_prefill_noalloc(P[0], 80 * 128, BF16, P[1], None, None, P[2], P[3], P[4], 1, T, 16, 48,
                                             128, 1.0, 1e-6, None, None, P[5], 48 * 128, P[6], 1e-6, P[7], None, F32,
                                             None)
    assert st == UNS
