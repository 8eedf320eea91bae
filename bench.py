"""Benchmark of the gated delta-rule layer on one MI355X.

One step = the full-layer prefill chain on T = 8192 tokens of one sequence with the layer's
shapes (16 key / 48 value heads of 128, hidden 5120): kernel-4 causal conv + SiLU + L2 norm of
q/k over the 10240 q|k|v channels -> chunked gated delta rule (chunk 64, fp32 state) -> gated
RMSNorm, the whole layer in one call (agnes_gdn_layer_prefill: conv, recurrence and norm, the
recurrence output never written).  `value` is tokens/s of K such steps timed back to back
between two synchronisations, each step on the next of four full copies of the inputs,
workspace and outputs (2.3 GB in all, several times the 256 MB last-level cache), so that no
step finds its data in a cache; the warm figure (the same buffers call after call) is reported
beside it.

The same run reports:
  * the same chain as two calls (agnes_gdn_prefill_fused, then the norm) and as three (conv,
    prefill, norm);
  * the whole-layer call on one sequence of 65536 tokens and on the packed batch of 32
    log-uniform sequences (251,984 tokens), each with its roofline;
  * the batched decode step (256 sequences, one token each, fp32 states updated in place) with
    its HBM roofline, and the fused decode step beside the three unfused calls it replaces;
  * the global attention layer's prefill (24 query / 4 KV heads of 256, T = 8192) and decode
    step (64 x 8191-token KV cache);
  * ceilings measured on this machine: the library's in-place HBM read-modify-write stream
    over 805 MB (the decode state's access pattern) and its register-resident bf16 matrix-core
    loop, beside a device-to-device copy and torch's bf16 GEMM; every roofline fraction is
    given against the vendor's peak and against the measured ceiling;
  * the fp64 oracle timed on the host cores (a prefill sample and one decode step).

Per-call durations are HIP events on the stream the library launches on (torch's current
stream); figures are medians of >= 20 calls unless said otherwise.  Inputs are synthetic and
seeded, resident in HBM before timing.

    python bench.py [--steps K] [--warmup W] [--decode-steps D] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "delta-layer prefill tokens/s (T=8192) + decode state HBM GB/s, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 matrix cores, TFLOP/s

T = 8192
HK, HV, D, CH = 16, 48, 128, 64
CCH = (2 * HK + HV) * D       # conv channels q | k | v
# Canonical chunked-recurrence FLOPs per token (WY/UT form, per 64-token chunk and key group:
# Gram K K^T and Q K^T, then per value head two C x C x d products for the WY factors, plus
# per value head three C x d x d state products and one C x C x d intra-chunk product).
FLOP_PER_CHUNK_GROUP = 2 * (2 * CH * CH * D + 3 * 2 * CH * CH * D) + 3 * 2 * (3 * CH * D * D + CH * CH * D)
FLOP_PER_TOKEN = FLOP_PER_CHUNK_GROUP * HK // CH                      # 7,602,176
STATE_BYTES = HV * D * D * 4                                          # one sequence's fp32 state
# whole-layer call per token: x in (q|k|v channels), g, beta, z in, y out (bf16)
LAYER_BYTES_PER_TOKEN = CCH * 2 + 2 * HV * 4 + HV * D * 2 * 2
LAYER_FIXED_BYTES = CCH * 4 * 2 + D * 2                               # conv and norm weights
LAYER_BYTES = T * LAYER_BYTES_PER_TOKEN + LAYER_FIXED_BYTES + STATE_BYTES  # + final state
PREFILL_FUSED_BYTES = T * (CCH * 2 + 2 * HV * 4 + HV * D * 2) + CCH * 4 * 2 + STATE_BYTES
CONV_BYTES = T * CCH * 2 * 2 + CCH * 4 * 2                            # x in, y out, weights
NORM_BYTES = T * HV * D * 2 * 3 + D * 2                               # o, z in, y out, weight
DECODE_B = 256
DECODE_STATE_BYTES = DECODE_B * HV * D * D * 4                        # 805 MB
DECODE_BYTES = DECODE_STATE_BYTES * 2 + DECODE_B * (2 * HK * D * 2 + HV * D * 2 + HV * D * 2 + 2 * HV * 4)
# fused decode: state read + write, x, conv history read + write, conv weights, z, y, g, beta, norm weight
FUSED_DECODE_BYTES = (DECODE_STATE_BYTES * 2 + DECODE_B * CCH * 2 + DECODE_B * CCH * 3 * 2 * 2
                      + CCH * 4 * 2 + DECODE_B * HV * D * 2 * 2 + DECODE_B * HV * 4 * 2 + D * 2)
CAL_BYTES = 256 << 20          # device-to-device copy of known size, for the HBM counter scale
NSETS = 4                      # rotating copies of the headline's buffers
# global attention layer (24 query / 4 KV heads of 256): QK^T and PV over the causal pairs,
# 2 x 256 multiply-adds each per query head
ATTN_HQ, ATTN_HKV, ATTN_D = 24, 4, 256
ATTN_FLOP = ATTN_HQ * 4 * ATTN_D * T * (T + 1) // 2
# attention decode: 64 entries with 8191 cached tokens each; per step the K and V caches of the
# 8192 keys are read once, plus q, gate, o rows and the new k, v rows
ATTN_DEC_B, ATTN_DEC_LEN = 64, 8192
ATTN_DEC_BYTES = (ATTN_DEC_B * ATTN_DEC_LEN * ATTN_HKV * ATTN_D * 2 * 2
                  + ATTN_DEC_B * ATTN_D * 2 * (3 * ATTN_HQ + 4 * ATTN_HKV))
MFMA_BLOCKS, MFMA_ITERS = 2048, 4096   # ceiling loop: 2048 x 4 waves x 4096 x 8 products

# HBM traffic per call from the committed counter summary (FETCH_SIZE and WRITE_SIZE runs, each
# scaled by the same counter on the calibration copy).  A figure is used only while the source
# file of its kernels still has the hash recorded with the counters.
PMC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_t8192_b256_pmc.md")
CSRC = os.path.join(ROOT, "gated_delta_rule_35_amd", "csrc")


def measured_traffic(name):
    """Bytes per call of `name` from the counter summary, or None if absent or stale."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"^traffic\s+" + re.escape(name) + r"\s+bytes=(\d+)\s+source=(\S+)\s+sha256=([0-9a-f]+)\s*$", text, re.M)
    if not m:
        return None
    try:
        digest = hashlib.sha256(open(os.path.join(CSRC, m.group(2)), "rb").read()).hexdigest()
    except OSError:
        return None
    return int(m.group(1)) if digest == m.group(3) else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--reps", type=int, default=20, help="calls per median of the side measurements")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=8192, help="tokens of the oracle prefill sample")
    return p.parse_args()


def to_dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def timed(torch, fn, reps, warmup=3, between=None):
    """Per-call durations (ms) of `reps` calls of fn(i) bracketed by events on the current
    stream; `between(i)` (untimed) runs before call i."""
    for i in range(warmup):
        if between:
            between(i)
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        if between:
            between(i)
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def host_info():
    info = {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "numpy": np.__version__,
            "machine": platform.machine()}
    try:
        import threadpoolctl
        blas = [d for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = blas[0].get("num_threads")
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return info


def cpu_baseline(cfg, ntok, dec):
    """The fp64 oracle (as it stands): the first `ntok` tokens of the same prefill chain, and one
    decode step of the 256-sequence decode workload (all 48 heads)."""
    import oracle
    from synth import decode_step_inputs
    t0 = time.perf_counter()
    x = cfg["x"][:ntok]
    y, _ = oracle.causal_conv(x, cfg["conv_w"], np.array([0, ntok]), None, l2_heads=32)
    q = y[:, :2048].reshape(ntok, HK, D)
    k = y[:, 2048:4096].reshape(ntok, HK, D)
    v = y[:, 4096:].reshape(ntok, HV, D)
    o, _ = oracle.recurrence(q, k, v, cfg["g"][:ntok], cfg["beta"][:ntok])
    oracle.gated_rmsnorm(o, cfg["z"][:ntok], cfg["norm_w"])
    dt = time.perf_counter() - t0
    d = decode_step_inputs(0, conv_input=False)
    picks = list(range(0, DECODE_B, 17))  # the 16 sequences the decode parity test follows
    t1 = time.perf_counter()
    oracle.decode_step(d["q"][picks], d["k"][picks], d["v"][picks], d["g"][picks], d["beta"][picks],
                       dec["state"][picks])
    dt_dec = time.perf_counter() - t1
    info = host_info()
    return {"value": ntok / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {ntok} of {T} tokens of the same chain (conv+L2, recurrence over all 48 value heads, "
                      f"gated RMSNorm), numpy fp64 token loop on one thread (numpy einsum, no BLAS call); "
                      f"{dt:.1f} s",
            "decode": {"value": len(picks) / dt_dec, "unit": "tokens/s", "seconds": round(dt_dec, 3),
                       "sample": f"one decode step of {len(picks)} of the 256 sequences of the decode workload "
                                 "(0, 17, .., 255), all 48 heads, fp64 oracle"},
            "host": info,
            "note": "the oracle is a correctness reference, not an optimised CPU kernel"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards by heads or by sequences with no collective inside the layer)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import gated_delta_rule_35_amd as gdn
    from synth import make_config, decode_step_inputs, varlen_lengths

    t_gen = time.perf_counter()
    cfg = make_config(1)
    dec = make_config(3)
    print(f"# inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    w = to_dev(cfg["conv_w"], torch)
    nw = to_dev(cfg["norm_w"], torch)

    # ---- headline: the whole-layer call on NSETS rotating copies of its buffers
    base = {k: to_dev(cfg[k], torch) for k in ("x", "g", "beta", "z")}
    wl_bytes = gdn.layer_prefill_workspace_size(1, T, HK, HV)
    sets = []
    for i in range(NSETS):
        s = {k: (v if i == 0 else v.clone()) for k, v in base.items()}
        s["ws"] = torch.empty(wl_bytes, dtype=torch.uint8, device="cuda")
        s["y"] = torch.empty((T, HV, D), dtype=torch.bfloat16, device="cuda")
        s["fin"] = torch.empty((1, HV, D, D), dtype=torch.float32, device="cuda")
        sets.append(s)

    def lstep(i):
        s = sets[i % NSETS]
        gdn.layer_prefill(s["x"], w, s["g"], s["beta"], cu, s["z"], nw, num_k_heads=HK, final_state=s["fin"],
                          y=s["y"], workspace=s["ws"])

    for i in range(args.warmup):
        lstep(i)
    torch.cuda.synchronize()
    levs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        levs[i][0].record()
        lstep(i)
        levs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cold = np.array([a.elapsed_time(b) for a, b in levs])
    value = T * args.steps / wall
    warm = timed(torch, lambda i: lstep(0), max(args.reps, 20))
    print(f"# headline: {wall * 1e3 / args.steps:.4f} ms/step cold, {np.median(warm):.4f} ms warm",
          file=sys.stderr, flush=True)

    # ---- the same chain as two calls and as three (set 0 buffers)
    s0 = sets[0]
    yconv = torch.empty((T, CCH), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, HV, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, HV, D), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((1, HV, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.prefill_workspace_size(1, T, HK, HV, torch.bfloat16), dtype=torch.uint8, device="cuda")
    q3, k3, v3 = (yconv[:, :2048].view(T, HK, D), yconv[:, 2048:4096].view(T, HK, D), yconv[:, 4096:].view(T, HV, D))
    ms_conv = timed(torch, lambda i: gdn.conv(s0["x"], w, y=yconv, cu_seqlens=cu, l2norm_heads=32), args.reps)
    ms_pre = timed(torch, lambda i: gdn.prefill_chunked(q3, k3, v3, s0["g"], s0["beta"], cu, final_state=fin, o=o,
                                                        workspace=ws), args.reps)
    ms_norm = timed(torch, lambda i: gdn.gated_rmsnorm(o, s0["z"], nw, y=out), args.reps)
    ms_fpre = timed(torch, lambda i: gdn.prefill_fused(s0["x"], w, s0["g"], s0["beta"], cu, num_k_heads=HK,
                                                       final_state=fin, o=o, workspace=ws), args.reps)
    del yconv, ws, q3, k3, v3

    # ---- measured ceilings
    buf = torch.ones(DECODE_STATE_BYTES // 4, dtype=torch.float32, device="cuda")
    ms_rmw = timed(torch, lambda i: gdn.ceiling_rmw_stream(buf), args.reps)
    dst = torch.empty_like(buf)
    ms_copy = timed(torch, lambda i: dst.copy_(buf), args.reps)
    del dst
    sink = torch.empty(MFMA_BLOCKS * 4, dtype=torch.float32, device="cuda")
    ms_mfma = timed(torch, lambda i: gdn.ceiling_mfma(sink, MFMA_BLOCKS, MFMA_ITERS), args.reps)
    mm_a = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    mm_b = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    ms_mm = timed(torch, lambda i: torch.matmul(mm_a, mm_b), args.reps)
    del mm_a, mm_b
    rmw_gbs = 2 * DECODE_STATE_BYTES / (np.median(ms_rmw) * 1e-3) / 1e9
    copy_gbs = 2 * DECODE_STATE_BYTES / (np.median(ms_copy) * 1e-3) / 1e9
    mfma_tf = MFMA_BLOCKS * 4 * MFMA_ITERS * 8 * 16384 / (np.median(ms_mfma) * 1e-3) / 1e12
    mm_tf = 2 * 8192 ** 3 / (np.median(ms_mm) * 1e-3) / 1e12
    # calibration copy of known size (untimed; read by the HBM counter runs)
    cal_src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst, buf
    print(f"# ceilings: rmw {rmw_gbs:.0f} GB/s, mfma {mfma_tf:.0f} TF/s", file=sys.stderr, flush=True)

    # ---- whole-layer call at 65536 tokens (one sequence) and on the 32-sequence varlen batch;
    # inputs drawn on the device (seeded) with the distributions of synth.layer_sequence_inputs
    def layer_case(lens, seed, init):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        n = int(sum(lens))
        c = {"x": (torch.randn((n, CCH), generator=gen, device="cuda") * 1.43).to(torch.bfloat16),
             "z": torch.randn((n, HV, D), generator=gen, device="cuda").to(torch.bfloat16),
             "g": -torch.nn.functional.softplus(torch.randn((n, HV), generator=gen, device="cuda")) * 0.05,
             "beta": torch.sigmoid(torch.randn((n, HV), generator=gen, device="cuda")),
             "w": (torch.rand((CCH, 4), generator=gen, device="cuda") - 0.5).to(torch.bfloat16),
             "cu": torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda"),
             "s0": torch.randn((len(lens), HV, D, D), generator=gen, device="cuda") * 0.01}
        if init == "alternate":
            c["s0"][0::2] = 0
        c["ws"] = torch.empty(gdn.layer_prefill_workspace_size(len(lens), n, HK, HV), dtype=torch.uint8,
                              device="cuda")
        c["y"] = torch.empty((n, HV, D), dtype=torch.bfloat16, device="cuda")
        c["fin"] = torch.empty((len(lens), HV, D, D), dtype=torch.float32, device="cuda")
        return c, n

    def layer_line(name, lens, seed, init, reps, traffic_key):
        c, n = layer_case(lens, seed, init)
        ms = timed(torch, lambda i: gdn.layer_prefill(c["x"], c["w"], c["g"], c["beta"], c["cu"], c["z"], nw,
                                                      num_k_heads=HK, initial_state=c["s0"], final_state=c["fin"],
                                                      y=c["y"], workspace=c["ws"]), reps)
        del c
        torch.cuda.empty_cache()
        med = float(np.median(ms))
        flops = FLOP_PER_TOKEN * n
        nbytes = n * LAYER_BYTES_PER_TOKEN + LAYER_FIXED_BYTES + 2 * STATE_BYTES * len(lens)
        tf = flops / (np.mean(ms) * 1e-3) / 1e12
        print(f"# {name}: {med:.3f} ms", file=sys.stderr, flush=True)
        return {"tokens": n, "sequences": len(lens), "ms_median": round(med, 4), "ms_mean": round(float(np.mean(ms)), 4),
                "tokens_per_s": round(n / (med * 1e-3), 1),
                "roofline": {"bound": "mfma", "kernel": "agnes_gdn_layer_prefill call", "achieved": round(tf, 2),
                             "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS, 4),
                             "frac_of_measured_ceiling": round(tf / mfma_tf, 4),
                             "traffic": measured_traffic(traffic_key),
                             "flops_per_launch": flops, "bytes_per_launch": nbytes,
                             "hbm_GBps_algorithmic": round(nbytes / (np.mean(ms) * 1e-3) / 1e9, 1)}}

    long_line = layer_line("layer T=65536", [65536], 2002, "normal", args.reps, "layer_prefill_t65536")
    vl = varlen_lengths(np.random.default_rng(1004))
    varlen_line = layer_line("layer varlen 32", [int(x) for x in vl], 2004, "alternate", args.reps,
                             "layer_prefill_varlen32")

    # ---- decode: 256 sequences, fp32 states in place (805 MB, larger than every cache)
    state = to_dev(dec["state"], torch)
    cache = to_dev(dec["conv_cache"], torch)
    cw = to_dev(dec["conv_w"], torch)
    ring = []
    for s in range(4):
        d = decode_step_inputs(s, gate_input=True)
        ring.append({kk: to_dev(vv, torch) for kk, vv in d.items()})
    yd = torch.empty((DECODE_B, CCH), dtype=torch.bfloat16, device="cuda")
    od = torch.empty((DECODE_B, HV, D), dtype=torch.bfloat16, device="cuda")
    yn = torch.empty((DECODE_B, HV, D), dtype=torch.bfloat16, device="cuda")
    nwd = to_dev(dec["norm_w"], torch)
    ms_dconv = timed(torch, lambda i: gdn.conv(ring[i % 4]["x"], cw, y=yd, cu_seqlens=None, conv_state=cache,
                                               l2norm_heads=32), args.decode_steps)
    ms_dec = timed(torch, lambda i: gdn.decode_step(ring[i % 4]["q"], ring[i % 4]["k"], ring[i % 4]["v"],
                                                    ring[i % 4]["g"], ring[i % 4]["beta"], state, o=od),
                   args.decode_steps)
    ms_dnorm = timed(torch, lambda i: gdn.gated_rmsnorm(od, ring[i % 4]["z"], nwd, y=yn), args.decode_steps)
    ms_fused = timed(torch, lambda i: gdn.decode_fused(ring[i % 4]["x"], cw, cache, ring[i % 4]["g"], ring[i % 4]["beta"],
                                                       ring[i % 4]["z"], nwd, state, num_k_heads=HK, y=yn),
                     args.decode_steps)
    dec_gbs = DECODE_BYTES / (np.mean(ms_dec) * 1e-3) / 1e9
    fused_gbs = FUSED_DECODE_BYTES / (np.mean(ms_fused) * 1e-3) / 1e9
    del state, cache, ring

    # ---- global attention prefill, T = 8192, one sequence
    from synth import attn_prefill_inputs
    ad = attn_prefill_inputs(np.random.default_rng(2001), [T], ATTN_HQ, ATTN_HKV, ATTN_D)
    aq, ak, av, ag = (to_dev(ad[n], torch) for n in ("q", "k", "v", "gate"))
    aqw, akw = to_dev(ad["qw"], torch), to_dev(ad["kw"], torch)
    ako = torch.empty((T, ATTN_HKV, ATTN_D), dtype=torch.bfloat16, device="cuda")
    ao = torch.empty((T, ATTN_HQ, ATTN_D), dtype=torch.bfloat16, device="cuda")
    aws = torch.empty(gdn.attn_prefill_workspace_size(1, T), dtype=torch.uint8, device="cuda")
    ms_attn = timed(torch, lambda i: gdn.attn_prefill(aq, ak, av, ag, aqw, akw, cu, k_out=ako, o=ao, workspace=aws),
                    args.reps)
    attn_tflops = ATTN_FLOP / (np.mean(ms_attn) * 1e-3) / 1e12
    del aq, ak, av, ag, ako, ao, aws

    # ---- global attention decode: 64 entries, 8191 cached tokens each
    from synth import attn_decode_inputs
    dd = attn_decode_inputs(np.random.default_rng(2002), [0] * ATTN_DEC_B, 1, ATTN_HQ, ATTN_HKV, ATTN_D)
    dq, dk, dv, dg = (to_dev(dd[n], torch) for n in ("q", "k", "v", "gate"))
    dkc = torch.randn((ATTN_DEC_B, ATTN_DEC_LEN, ATTN_HKV, ATTN_D), device="cuda").to(torch.bfloat16)
    dvc = (torch.randn((ATTN_DEC_B, ATTN_DEC_LEN, ATTN_HKV, ATTN_D), device="cuda") * 1.43).to(torch.bfloat16)
    dlens = torch.full((ATTN_DEC_B,), ATTN_DEC_LEN - 1, dtype=torch.int32, device="cuda")
    dao = torch.empty((ATTN_DEC_B, ATTN_HQ, ATTN_D), dtype=torch.bfloat16, device="cuda")
    dws = torch.empty(gdn.attn_decode_workspace_size(ATTN_DEC_B, ATTN_HQ, ATTN_HKV, ATTN_DEC_LEN), dtype=torch.uint8,
                      device="cuda")
    ms_adec = timed(torch, lambda i: gdn.attn_decode(dq, dk, dv, dg, aqw, akw, dkc, dvc, dlens, o=dao, workspace=dws),
                    args.decode_steps)
    adec_gbs = ATTN_DEC_BYTES / (np.mean(ms_adec) * 1e-3) / 1e9
    del dkc, dvc

    med = lambda a: round(float(np.median(a)), 4)  # noqa: E731
    layer_ms = float(np.mean(cold))
    layer_tflops = FLOP_PER_TOKEN * T / (layer_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "delta-layer prefill chain, T=8192, 1 sequence: conv(k=4)+SiLU+L2 -> "
                               "chunked gated delta rule (chunk 64) -> gated RMSNorm, the whole layer in "
                               "one call (agnes_gdn_layer_prefill)",
                   "T": T, "num_k_heads": HK, "num_v_heads": HV, "head_dim": D, "chunk": CH,
                   "io_dtype": "bf16", "matrix_core_operands": "fp16", "accumulate": "fp32",
                   "state": "fp32", "parallelism": "none (1 GPU)"},
        "headline_timing": {
            "mode": f"{args.steps} calls back to back on {NSETS} rotating copies of inputs, workspace and outputs "
                    f"({NSETS * (2 * T * CCH + 4 * T * HV * D + 8 * T * HV + wl_bytes) / 1e9:.1f} GB, several times "
                    "the 256 MB last-level cache), bracketed by synchronisations",
            "call_ms_median_cold": med(cold), "call_ms_mean_cold": round(layer_ms, 4),
            "call_ms_median_warm": med(warm), "tokens_per_s_warm": round(T / (np.median(warm) * 1e-3), 1)},
        "kernels_ms": {"layer_prefill": med(cold)},
        "two_call_chain": {"prefill_fused": med(ms_fpre), "gated_rmsnorm": med(ms_norm),
                           "tokens_per_s": round(T / ((np.median(ms_fpre) + np.median(ms_norm)) * 1e-3), 1),
                           "prefill_fused_TFLOPs": round(FLOP_PER_TOKEN * T / (np.median(ms_fpre) * 1e-3) / 1e12, 2),
                           "prefill_fused_traffic": measured_traffic("prefill_fused"),
                           "prefill_fused_GBps_algorithmic": round(PREFILL_FUSED_BYTES / (np.median(ms_fpre) * 1e-3) / 1e9, 1)},
        "unfused_chain": {"conv": med(ms_conv), "prefill_chunked": med(ms_pre), "gated_rmsnorm": med(ms_norm),
                          "tokens_per_s": round(T / ((np.median(ms_conv) + np.median(ms_pre) + np.median(ms_norm)) * 1e-3), 1),
                          "prefill_chunked_TFLOPs": round(FLOP_PER_TOKEN * T / (np.median(ms_pre) * 1e-3) / 1e12, 2),
                          "prefill_chunked_traffic": measured_traffic("prefill_chunked")},
        "roofline": {"bound": "mfma",
                     "kernel": "agnes_gdn_layer_prefill call (chunk_offsets + prep + scan launches)",
                     "achieved": round(layer_tflops, 2),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(layer_tflops / MFMA_PEAK_TFLOPS, 4),
                     "frac_of_measured_ceiling": round(layer_tflops / mfma_tf, 4),
                     "traffic": measured_traffic("layer_prefill"), "flops_per_launch": FLOP_PER_TOKEN * T,
                     "bytes_per_launch": LAYER_BYTES,
                     "hbm_GBps_algorithmic": round(LAYER_BYTES / (layer_ms * 1e-3) / 1e9, 1)},
        "layer_prefill_t65536": long_line,
        "layer_prefill_varlen32": varlen_line,
        "ceilings": {"rmw_stream_GBps": round(rmw_gbs, 1), "rmw_stream_bytes": 2 * DECODE_STATE_BYTES,
                     "rmw_stream_frac_of_spec": round(rmw_gbs / HBM_PEAK_GBS, 4),
                     "d2d_copy_GBps": round(copy_gbs, 1),
                     "mfma_bf16_TFLOPs": round(mfma_tf, 1), "mfma_frac_of_spec": round(mfma_tf / MFMA_PEAK_TFLOPS, 4),
                     "torch_matmul_bf16_8192_TFLOPs": round(mm_tf, 1),
                     "note": "rmw: the library's in-place read+write stream over 805 MB (agnes_gdn_ceiling_rmw_stream); "
                             "mfma: its register-resident bf16 16x16x32 loop on every SIMD (agnes_gdn_ceiling_mfma); "
                             "copy and matmul: torch (device-to-device copy, hipBLASLt GEMM), for reference"},
        "streaming_kernels": {
            "conv_GBps": round(CONV_BYTES / (np.median(ms_conv) * 1e-3) / 1e9, 1),
            "gated_rmsnorm_GBps": round(NORM_BYTES / (np.median(ms_norm) * 1e-3) / 1e9, 1)},
        "decode": {"batch": DECODE_B, "steps": args.decode_steps, "us_per_step": round(float(np.median(ms_dec)) * 1e3, 2),
                   "tokens_per_s": round(DECODE_B / (np.median(ms_dec) * 1e-3), 1),
                   "conv_decode_us": round(float(np.median(ms_dconv)) * 1e3, 2),
                   "roofline": {"bound": "hbm", "kernel": "decode_step_kernel", "achieved": round(dec_gbs, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                                "frac_of_measured_ceiling": round(dec_gbs / rmw_gbs, 4),
                                "traffic": measured_traffic("decode_step"), "bytes_per_launch": DECODE_BYTES}},
        "decode_fused": {"batch": DECODE_B, "steps": args.decode_steps,
                         "us_per_step": round(float(np.median(ms_fused)) * 1e3, 2),
                         "tokens_per_s": round(DECODE_B / (np.median(ms_fused) * 1e-3), 1),
                         "unfused_conv_decode_norm_us": round(float(np.median(ms_dconv) + np.median(ms_dec)
                                                                    + np.median(ms_dnorm)) * 1e3, 2),
                         "unfused_norm_us": round(float(np.median(ms_dnorm)) * 1e3, 2),
                         "roofline": {"bound": "hbm", "kernel": "decode_fused_kernel", "achieved": round(fused_gbs, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(fused_gbs / HBM_PEAK_GBS, 4),
                                      "frac_of_measured_ceiling": round(fused_gbs / rmw_gbs, 4),
                                      "traffic": measured_traffic("decode_fused"),
                                      "bytes_per_launch": FUSED_DECODE_BYTES}},
        "attention_prefill": {"T": T, "num_q_heads": ATTN_HQ, "num_kv_heads": ATTN_HKV, "head_dim": ATTN_D,
                              "ms": med(ms_attn), "tokens_per_s": round(T / (np.median(ms_attn) * 1e-3), 1),
                              "roofline": {"bound": "mfma",
                                           "kernel": "agnes_attn_prefill call (offsets + k prep + attention launches)",
                                           "achieved": round(attn_tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                                           "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_PEAK_TFLOPS, 4),
                                           "frac_of_measured_ceiling": round(attn_tflops / mfma_tf, 4),
                                           "flops_per_launch": ATTN_FLOP, "operands": "bf16"}},
        "attention_decode": {"batch": ATTN_DEC_B, "cached_tokens": ATTN_DEC_LEN - 1, "steps": args.decode_steps,
                             "us_per_step": round(float(np.median(ms_adec)) * 1e3, 2),
                             "tokens_per_s": round(ATTN_DEC_B / (np.median(ms_adec) * 1e-3), 1),
                             "roofline": {"bound": "hbm",
                                          "kernel": "agnes_attn_decode call (prep + split-K attention + combine)",
                                          "achieved": round(adec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                          "frac": round(adec_gbs / HBM_PEAK_GBS, 4),
                                          "frac_of_measured_ceiling": round(adec_gbs / rmw_gbs, 4),
                                          "bytes_per_launch": ATTN_DEC_BYTES,
                                          "note": "a read stream (the cache) against a read+write ceiling, "
                                                  "so the fraction may pass 1"}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_tokens, dec)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
