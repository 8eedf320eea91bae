"""Benchmark of the gated delta-rule layer on one MI355X.

One step = the full-layer prefill chain on T = 8192 tokens of one sequence with the layer's
shapes (16 key / 48 value heads of 128, hidden 5120): kernel-4 causal conv + SiLU + L2 norm of
q/k over the 10240 q|k|v channels -> chunked gated delta rule (chunk 64, fp32 state) -> gated
RMSNorm.  `value` is tokens/s of that chain as the library runs it fastest: the whole layer in
one call (agnes_gdn_layer_prefill: conv, recurrence and norm, the recurrence output never
written).  The same chain as two calls (agnes_gdn_prefill_fused, then the norm) and as three
(conv, prefill, norm) is timed beside it.  The same run also times the batched decode step
(256 sequences, one token each, fp32 states updated in place) and reports its state HBM GB/s,
and the fused decode step (conv-history update + conv + L2 + recurrence + gated norm in one
launch) beside the three unfused calls it replaces, and the prefill of the model's global
attention layer (24 query / 4 KV heads of 256, T = 8192) with its matrix-core roofline, and
that layer's decode step over a 64 x 8191-token bf16 KV cache with its HBM roofline.

Inputs are synthetic (seeded), generated on the host and resident in HBM before timing.

    python bench.py [--steps K] [--warmup W] [--decode-steps D] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
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
# Canonical chunked-recurrence FLOPs per token (WY/UT form, per 64-token chunk and key group:
# Gram K K^T and Q K^T, then per value head two C x C x d products for the WY factors, plus
# per value head three C x d x d state products and one C x C x d intra-chunk product).
FLOP_PER_CHUNK_GROUP = 2 * (2 * CH * CH * D + 3 * 2 * CH * CH * D) + 3 * 2 * (3 * CH * D * D + CH * CH * D)
FLOP_PER_TOKEN = FLOP_PER_CHUNK_GROUP * HK // CH                      # 7,602,176
PREFILL_BYTES = T * (2 * HK * D * 2 + HV * D * 2 + HV * D * 2 + 2 * HV * 4) + HV * D * D * 4  # q,k,v,o,g,beta + final state
# fused call: x (q|k|v channels) in, conv weights, g, beta, o out, final state
PREFILL_FUSED_BYTES = T * (10240 * 2 + 2 * HV * 4 + HV * D * 2) + 10240 * 4 * 2 + HV * D * D * 4
# whole-layer call: x in, conv weights, g, beta, z in, y out, norm weight, final state
LAYER_BYTES = T * (10240 * 2 + 2 * HV * 4 + HV * D * 2 * 2) + 10240 * 4 * 2 + D * 2 + HV * D * D * 4
CONV_BYTES = T * 10240 * 2 * 2 + 10240 * 4 * 2                        # x in, y out, weights
NORM_BYTES = T * HV * D * 2 * 3 + D * 2                               # o, z in, y out, weight
DECODE_B = 256
DECODE_BYTES = DECODE_B * HV * D * D * 4 * 2 + DECODE_B * (2 * HK * D * 2 + HV * D * 2 + HV * D * 2 + 2 * HV * 4)
# fused decode: state read + write, x, conv history read + write, conv weights, z, y, g, beta, norm weight
FUSED_DECODE_BYTES = (DECODE_B * HV * D * D * 4 * 2 + DECODE_B * 10240 * 2 + DECODE_B * 10240 * 3 * 2 * 2
                      + 10240 * 4 * 2 + DECODE_B * HV * D * 2 * 2 + DECODE_B * HV * 4 * 2 + D * 2)
CAL_BYTES = 256 << 20          # device-to-device copy of known size, for the HBM counter scale
# global attention layer (24 query / 4 KV heads of 256): QK^T and PV over the causal pairs,
# 2 x 256 multiply-adds each per query head
ATTN_HQ, ATTN_HKV, ATTN_D = 24, 4, 256
ATTN_FLOP = ATTN_HQ * 4 * ATTN_D * T * (T + 1) // 2
# attention decode: 64 entries with 8191 cached tokens each; per step the K and V caches of the
# 8192 keys are read once, plus q, gate, o rows and the new k, v rows
ATTN_DEC_B, ATTN_DEC_LEN = 64, 8192
ATTN_DEC_BYTES = (ATTN_DEC_B * ATTN_DEC_LEN * ATTN_HKV * ATTN_D * 2 * 2
                  + ATTN_DEC_B * ATTN_D * 2 * (3 * ATTN_HQ + 4 * ATTN_HKV))

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
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=8192, help="tokens of the oracle CPU sample")
    return p.parse_args()


def to_dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def cpu_baseline(cfg, ntok):
    """The fp64 oracle (as it stands) on the first `ntok` tokens of the same chain."""
    import oracle
    t0 = time.perf_counter()
    x = cfg["x"][:ntok]
    y, _ = oracle.causal_conv(x, cfg["conv_w"], np.array([0, ntok]), None, l2_heads=32)
    q = y[:, :2048].reshape(ntok, HK, D)
    k = y[:, 2048:4096].reshape(ntok, HK, D)
    v = y[:, 4096:].reshape(ntok, HV, D)
    o, _ = oracle.recurrence(q, k, v, cfg["g"][:ntok], cfg["beta"][:ntok])
    oracle.gated_rmsnorm(o, cfg["z"][:ntok], cfg["norm_w"])
    dt = time.perf_counter() - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {ntok} of {T} tokens of the same chain (conv+L2, recurrence over all 48 "
                      f"value heads, gated RMSNorm), numpy fp64, single-threaded token loop; "
                      f"{dt:.1f} s; host cpu_count={os.cpu_count()}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards by heads or by sequences with no collective inside the layer)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import gated_delta_rule_35_amd as gdn
    from synth import make_config, decode_step_inputs

    t_gen = time.perf_counter()
    cfg = make_config(1)
    dec = make_config(3)
    print(f"# inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    x = to_dev(cfg["x"], torch)
    w = to_dev(cfg["conv_w"], torch)
    g = to_dev(cfg["g"], torch)
    beta = to_dev(cfg["beta"], torch)
    z = to_dev(cfg["z"], torch)
    nw = to_dev(cfg["norm_w"], torch)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    y = torch.empty((T, 10240), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, HV, D), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((1, HV, D, D), dtype=torch.float32, device="cuda")
    out = torch.empty((T, HV, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.prefill_workspace_size(1, T, HK, HV, torch.bfloat16), dtype=torch.uint8, device="cuda")
    ws_l = torch.empty(gdn.layer_prefill_workspace_size(1, T, HK, HV), dtype=torch.uint8, device="cuda")
    q = y[:, :2048].view(T, HK, D)
    k = y[:, 2048:4096].view(T, HK, D)
    v = y[:, 4096:].view(T, HV, D)

    def step(ev=None):  # the chain as three calls
        if ev is not None:
            ev[0].record()
        gdn.conv(x, w, y=y, cu_seqlens=cu, l2norm_heads=32)
        if ev is not None:
            ev[1].record()
        gdn.prefill_chunked(q, k, v, g, beta, cu, final_state=fin, o=o, workspace=ws)
        if ev is not None:
            ev[2].record()
        gdn.gated_rmsnorm(o, z, nw, y=out)
        if ev is not None:
            ev[3].record()

    def fstep(ev=None):  # conv inside the prefill call, then the norm
        if ev is not None:
            ev[0].record()
        gdn.prefill_fused(x, w, g, beta, cu, num_k_heads=HK, final_state=fin, o=o, workspace=ws)
        if ev is not None:
            ev[1].record()
        gdn.gated_rmsnorm(o, z, nw, y=out)
        if ev is not None:
            ev[2].record()

    def lstep(ev=None):  # the whole layer in one call
        if ev is not None:
            ev[0].record()
        gdn.layer_prefill(x, w, g, beta, cu, z, nw, num_k_heads=HK, final_state=fin, y=out, workspace=ws_l)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
        fstep()
        lstep()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_conv = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    ms_pre = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    ms_norm = np.mean([e[2].elapsed_time(e[3]) for e in evs])
    ms_step = np.mean([e[0].elapsed_time(e[3]) for e in evs])
    fevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        fstep(fevs[i])
    torch.cuda.synchronize()
    ms_fpre = np.mean([e[0].elapsed_time(e[1]) for e in fevs])
    ms_fnorm = np.mean([e[1].elapsed_time(e[2]) for e in fevs])
    ms_fstep = np.mean([e[0].elapsed_time(e[2]) for e in fevs])
    # headline: K whole-layer calls, bracketed by synchronisations
    levs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        lstep(levs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_layer = np.mean([e[0].elapsed_time(e[1]) for e in levs])
    value = T * args.steps / wall

    # ---- calibration copy of known size (untimed; read by the HBM counter runs)
    cal_src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    # ---- decode: 256 sequences, fp32 states in place
    state = to_dev(dec["state"], torch)
    cache = to_dev(dec["conv_cache"], torch)
    cw = to_dev(dec["conv_w"], torch)
    ring = []
    for s in range(4):
        d = decode_step_inputs(s, gate_input=True)
        ring.append({kk: to_dev(vv, torch) for kk, vv in d.items()})
    yd = torch.empty((DECODE_B, 10240), dtype=torch.bfloat16, device="cuda")
    od = torch.empty((DECODE_B, HV, D), dtype=torch.bfloat16, device="cuda")
    yn = torch.empty((DECODE_B, HV, D), dtype=torch.bfloat16, device="cuda")
    nwd = to_dev(dec["norm_w"], torch)

    def dstep(i, ev=None):
        d = ring[i % len(ring)]
        if ev is not None:
            ev[0].record()
        gdn.conv(d["x"], cw, y=yd, cu_seqlens=None, conv_state=cache, l2norm_heads=32)
        if ev is not None:
            ev[1].record()
        gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, o=od)
        if ev is not None:
            ev[2].record()
        gdn.gated_rmsnorm(od, d["z"], nwd, y=yn)
        if ev is not None:
            ev[3].record()

    def fstep(i, ev=None):
        d = ring[i % len(ring)]
        if ev is not None:
            ev[0].record()
        gdn.decode_fused(d["x"], cw, cache, d["g"], d["beta"], d["z"], nwd, state, num_k_heads=HK, y=yn)
        if ev is not None:
            ev[1].record()

    for i in range(5):
        dstep(i)
    torch.cuda.synchronize()
    devs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.decode_steps)]
    for i in range(args.decode_steps):
        dstep(i, devs[i])
    torch.cuda.synchronize()
    ms_dconv = np.mean([e[0].elapsed_time(e[1]) for e in devs])
    ms_dec = np.mean([e[1].elapsed_time(e[2]) for e in devs])
    ms_dnorm = np.mean([e[2].elapsed_time(e[3]) for e in devs])
    ms_dchain = np.mean([e[0].elapsed_time(e[3]) for e in devs])
    dec_gbs = DECODE_BYTES / (ms_dec * 1e-3) / 1e9
    for i in range(5):
        fstep(i)
    torch.cuda.synchronize()
    fevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.decode_steps)]
    for i in range(args.decode_steps):
        fstep(i, fevs[i])
    torch.cuda.synchronize()
    ms_fused = np.mean([e[0].elapsed_time(e[1]) for e in fevs])
    fused_gbs = FUSED_DECODE_BYTES / (ms_fused * 1e-3) / 1e9

    # ---- global attention prefill, T = 8192, one sequence
    from synth import attn_prefill_inputs
    ad = attn_prefill_inputs(np.random.default_rng(2001), [T], ATTN_HQ, ATTN_HKV, ATTN_D)
    aq, ak, av, ag = (to_dev(ad[n], torch) for n in ("q", "k", "v", "gate"))
    aqw, akw = to_dev(ad["qw"], torch), to_dev(ad["kw"], torch)
    acu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    ako = torch.empty((T, ATTN_HKV, ATTN_D), dtype=torch.bfloat16, device="cuda")
    ao = torch.empty((T, ATTN_HQ, ATTN_D), dtype=torch.bfloat16, device="cuda")
    aws = torch.empty(gdn.attn_prefill_workspace_size(1, T), dtype=torch.uint8, device="cuda")

    def astep():
        gdn.attn_prefill(aq, ak, av, ag, aqw, akw, acu, k_out=ako, o=ao, workspace=aws)

    for _ in range(max(args.warmup, 1)):
        astep()
    torch.cuda.synchronize()
    aevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        aevs[i][0].record()
        astep()
        aevs[i][1].record()
    torch.cuda.synchronize()
    ms_attn = np.mean([e[0].elapsed_time(e[1]) for e in aevs])
    attn_tflops = ATTN_FLOP / (ms_attn * 1e-3) / 1e12
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

    def adstep():
        gdn.attn_decode(dq, dk, dv, dg, aqw, akw, dkc, dvc, dlens, o=dao, workspace=dws)

    for _ in range(3):
        adstep()
    torch.cuda.synchronize()
    devs2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.decode_steps)]
    for i in range(args.decode_steps):
        devs2[i][0].record()
        adstep()
        devs2[i][1].record()
    torch.cuda.synchronize()
    ms_adec = np.mean([e[0].elapsed_time(e[1]) for e in devs2])
    adec_gbs = ATTN_DEC_BYTES / (ms_adec * 1e-3) / 1e9
    del dkc, dvc

    layer_tflops = FLOP_PER_TOKEN * T / (ms_layer * 1e-3) / 1e12
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
        "kernels_ms": {"layer_prefill": round(ms_layer, 4)},
        "two_call_chain": {"prefill_fused": round(ms_fpre, 4), "gated_rmsnorm": round(ms_fnorm, 4),
                           "chain_events": round(ms_fstep, 4), "tokens_per_s": round(T / (ms_fstep * 1e-3), 1),
                           "prefill_fused_TFLOPs": round(FLOP_PER_TOKEN * T / (ms_fpre * 1e-3) / 1e12, 2),
                           "prefill_fused_traffic": measured_traffic("prefill_fused"),
                           "prefill_fused_GBps_algorithmic": round(PREFILL_FUSED_BYTES / (ms_fpre * 1e-3) / 1e9, 1)},
        "unfused_chain": {"conv": round(ms_conv, 4), "prefill_chunked": round(ms_pre, 4),
                          "gated_rmsnorm": round(ms_norm, 4), "chain_events": round(ms_step, 4),
                          "tokens_per_s": round(T / (ms_step * 1e-3), 1),
                          "prefill_chunked_TFLOPs": round(FLOP_PER_TOKEN * T / (ms_pre * 1e-3) / 1e12, 2),
                          "prefill_chunked_traffic": measured_traffic("prefill_chunked")},
        "roofline": {"bound": "mfma",
                     "kernel": "agnes_gdn_layer_prefill call (chunk_offsets + prep + scan launches)",
                     "achieved": round(layer_tflops, 2),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(layer_tflops / MFMA_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("layer_prefill"), "flops_per_launch": FLOP_PER_TOKEN * T,
                     "bytes_per_launch": LAYER_BYTES,
                     "hbm_GBps_algorithmic": round(LAYER_BYTES / (ms_layer * 1e-3) / 1e9, 1)},
        "streaming_kernels": {
            "conv_GBps": round(CONV_BYTES / (ms_conv * 1e-3) / 1e9, 1),
            "gated_rmsnorm_GBps": round(NORM_BYTES / (ms_norm * 1e-3) / 1e9, 1)},
        "decode": {"batch": DECODE_B, "steps": args.decode_steps, "us_per_step": round(ms_dec * 1e3, 2),
                   "tokens_per_s": round(DECODE_B / (ms_dec * 1e-3), 1),
                   "conv_decode_us": round(ms_dconv * 1e3, 2),
                   "roofline": {"bound": "hbm", "kernel": "decode_step_kernel", "achieved": round(dec_gbs, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                                "traffic": measured_traffic("decode_step"), "bytes_per_launch": DECODE_BYTES}},
        "decode_fused": {"batch": DECODE_B, "steps": args.decode_steps, "us_per_step": round(ms_fused * 1e3, 2),
                         "tokens_per_s": round(DECODE_B / (ms_fused * 1e-3), 1),
                         "unfused_conv_decode_norm_us": round(ms_dchain * 1e3, 2),
                         "unfused_norm_us": round(ms_dnorm * 1e3, 2),
                         "roofline": {"bound": "hbm", "kernel": "decode_fused_kernel", "achieved": round(fused_gbs, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(fused_gbs / HBM_PEAK_GBS, 4),
                                      "traffic": measured_traffic("decode_fused"),
                                      "bytes_per_launch": FUSED_DECODE_BYTES}},
        "attention_prefill": {"T": T, "num_q_heads": ATTN_HQ, "num_kv_heads": ATTN_HKV, "head_dim": ATTN_D,
                              "ms": round(ms_attn, 4), "tokens_per_s": round(T / (ms_attn * 1e-3), 1),
                              "roofline": {"bound": "mfma",
                                           "kernel": "agnes_attn_prefill call (offsets + k prep + attention launches)",
                                           "achieved": round(attn_tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                                           "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_PEAK_TFLOPS, 4),
                                           "flops_per_launch": ATTN_FLOP, "operands": "bf16"}},
        "attention_decode": {"batch": ATTN_DEC_B, "cached_tokens": ATTN_DEC_LEN - 1, "steps": args.decode_steps,
                             "us_per_step": round(ms_adec * 1e3, 2),
                             "tokens_per_s": round(ATTN_DEC_B / (ms_adec * 1e-3), 1),
                             "roofline": {"bound": "hbm",
                                          "kernel": "agnes_attn_decode call (prep + split-K attention + combine)",
                                          "achieved": round(adec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                          "frac": round(adec_gbs / HBM_PEAK_GBS, 4),
                                          "bytes_per_launch": ATTN_DEC_BYTES}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
