#!/usr/bin/env python3
"""Throughput benchmark for the differential-attention hot path on one MI355X.

Headline workload: DIFF V1 causal prefill, bf16 inputs / fp32 accumulation,
batch 4 x 12 heads x 4096 tokens, q/k head dim 128, v head dim 256
(d_model 3072), evaluated for layers l = 1..28 with lambda = lambda_init(l).
One step = the 28 layer calls on one synthetic batch; the metric is
algorithmic TFLOP/s (causal lower triangle, diagonal included).

The other hot-path kernels are timed in the same run (``secondary``):
V2 GQA causal prefill (B2, Hq64/Hkv8, T8192, d128), V2 packed varlen prefill
(65536 tokens in 8 sequences, and in 2048 sequences of 32), the V2 decode
step (B64 and B1, 32768-entry cache, Hq64/Hkv8, d128, metric HBM GB/s), the
V1 decode step (B32, 32768-entry cache, H12, d128/dv256, GB/s), the V2
backward on the prefill and packed workloads (2x the forward's FLOP: dP and
dV are formed once per head pair) and the V1 backward on the headline
workload, and the two projections either side of the V2 attention on its
tokens (coefficient logits, GB/s; output projection, TFLOP/s).  Inputs are
synthetic, seeded, already resident in HBM when timing starts.  Every timed
leg reports the mean over back-to-back calls and the median and minimum of
the per-call times (HIP events on the launch stream).

The fp64 CPU oracle is timed on bounded samples of the headline, V2 prefill,
packed prefill and decode workloads on this host (``cpu_baseline``, and
``cpu_baseline`` inside those secondary legs).

Every leg's untimed warm-up is its W calls (steps for the headline) and then
more until 100 ms of wall time have passed, so the timed calls run at the
clocks of sustained load; the headline then times exactly K steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]
       [--no-cpu-baseline] [--only LEG]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

LEGS = ["v1", "v2", "varlen", "varlen_short", "decode", "decode_b1", "v1dec", "bwd", "vbwd",
        "v1bwd", "lproj", "proj", "gda", "gda_dec"]

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "differential_softmax_attention_diffattn_amd", "csrc")
# kernel sources behind each timed workload (the HBM-traffic record is void once they change)
_V2P = ("v2_prefill.hip", "varlen.h", "device_common.h", "kernels.h")
_V2B = ("v2_backward.hip", "varlen.h", "bwd_common.h", "device_common.h", "kernels.h")
SOURCES = {
    "v1": ("v1_prefill.hip", "device_common.h", "kernels.h"),
    "v2": _V2P,
    "varlen": _V2P,
    "varlen_short": _V2P,
    "decode": ("v2_decode.hip", "device_common.h", "kernels.h"),
    "decode_b1": ("v2_decode.hip", "device_common.h", "kernels.h"),
    "gda": _V2P,
    "gda_dec": ("v2_decode.hip", "device_common.h", "kernels.h"),
    "bwd": _V2B,
    "vbwd": _V2B,
    "v1dec": ("v1_decode.hip", "device_common.h", "kernels.h"),
    "v1bwd": ("v1_backward.hip", "bwd_common.h", "device_common.h", "kernels.h"),
    "proj": ("proj.hip", "device_common.h", "kernels.h"),
    "lproj": ("proj.hip", "device_common.h", "kernels.h"),
}


def kernel_digest(which: str) -> str:
    """sha256 over the kernel sources of one workload (file order fixed)."""
    import hashlib

    h = hashlib.sha256()
    for name in SOURCES[which]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def hbm_traffic(which: str, workload: str):
    """HBM bytes per call from the committed counter record, or None.

    profiles/<workload>_hbm_traffic.txt holds FETCH_SIZE / WRITE_SIZE per
    dispatch (rocprofv3 --pmc, KiB) for the call's kernels, scaled by the
    factors a plain copy of known size gives, and the digest of the kernel
    sources they were taken with.  A record taken with other sources is not
    used (the kernels have changed since).
    """
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_sources_sha256") != kernel_digest(which):
        return None
    try:
        return int(float(rec["hbm_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def v1_flops(B, T, H, d, dv):
    return 2.0 * (d + dv) * T * (T + 1) * B * H


def v2_flops_seq(n, Hq, d):
    return 2.0 * d * n * (n + 1) * Hq


def v2_bwd_flops_seq(n, Hq, d):
    # per (query, key) pair and pair of heads: S_e, S_o, dP (shared: the odd
    # head's is -sigma times it), dV (one product of P_e - sigma P_o), dQ_e,
    # dQ_o, dK_e, dK_o: 8 products of 2d = 2x the forward's 2 per head
    return 2.0 * v2_flops_seq(n, Hq, d)


def v1_bwd_flops(B, T, H, d, dv):
    # per (query, key) pair and head: S1, S2, dQ1, dQ2, dK1, dK2 (2d each) and
    # dP = dz V^T, dV = (P1 - lambda P2)^T dz (2dv each), causal lower triangle
    return (12.0 * d + 4.0 * dv) * T * (T + 1) / 2 * B * H


def decode_bytes(B, S, Hkv, d):
    return 2.0 * B * S * Hkv * d * 2  # K and V once, bf16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def warm_up(fn, calls, min_ms=100.0):
    """Untimed warm-up: ``calls`` calls of ``fn``, then more until at least
    ``min_ms`` of wall time has passed since the start, so the timed calls that
    follow run at the clocks of sustained load (the first tens of milliseconds
    on an idle GPU run measurably slower)."""
    import torch

    t0 = time.perf_counter()
    for _ in range(calls):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        torch.cuda.synchronize()


def time_calls(fn, iters, stream):
    """Milliseconds per call of ``fn``, ``iters`` calls back to back, with HIP
    events on ``stream`` between the calls: the mean over the whole run and the
    median and minimum of the per-call times."""
    import torch

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    evs[0].record(stream)
    for i in range(iters):
        fn()
        evs[i + 1].record(stream)
    evs[-1].synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(iters)]
    return {"mean": evs[0].elapsed_time(evs[-1]) / iters, "median": statistics.median(per),
            "min": min(per)}


def rate(work, ms):
    """work per second from milliseconds, in tera (FLOP) or giga (bytes) units by caller."""
    return work / (ms * 1e-3)


def timing_fields(t, work, unit_scale, unit_key):
    """mean/median/min milliseconds and the rate at each."""
    return {"ms": round(t["mean"], 4), "ms_median": round(t["median"], 4),
            "ms_min": round(t["min"], 4), unit_key: round(rate(work, t["mean"]) / unit_scale, 2),
            f"{unit_key}_median": round(rate(work, t["median"]) / unit_scale, 2),
            f"{unit_key}_best": round(rate(work, t["min"]) / unit_scale, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=LEGS, default=None)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "the kernels would shard by head (V1) or KV head (V2) with no communication",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import differential_softmax_attention_diffattn_amd as da
    from differential_softmax_attention_diffattn_amd import inputs as inp

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cpu = not args.no_cpu_baseline
    result = {}
    secondary = {}

    def want(leg):
        return args.only == leg or (args.only is None and (leg == "v1" or not args.no_secondary))

    # ------------------------------------------------------------------ V1 (headline)
    if want("v1"):
        w = inp.V1_BF16
        log(f"[bench] generating {w.name}")
        x = inp.v1_inputs(w, device=dev)
        out = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device=dev)
        ws = torch.empty(da.v1_workspace_bytes(w.B, w.T, w.H, w.d, w.dv, torch.bfloat16),
                         dtype=torch.uint8, device=dev)
        lams = [da.lambda_init(l) for l in w.layers]

        def v1_call(li):
            da.v1_fwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], li, li, w.eps, out=out,
                      workspace=ws)

        def step():
            for li in lams:
                v1_call(li)

        warm_up(step, args.warmup)
        log(f"[bench] timing {args.steps} steps x {len(lams)} layer calls")
        t0 = time.perf_counter()
        tm = time_calls(step, args.steps, stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = tm["mean"]
        flop_call = v1_flops(w.B, w.T, w.H, w.d, w.dv)
        flop_step = flop_call * len(lams)
        tflops = flop_step / (ms_step * 1e-3) / 1e12
        ms_call = ms_step / len(lams)
        achieved = flop_call / (ms_call * 1e-3) / 1e12
        result = {
            "metric": "diff-attn prefill TFLOP/s (% bf16 MFMA peak); V2 decode HBM GB/s (% peak)",
            "value": round(tflops, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4),
            "ms_per_step_median": round(tm["median"], 4),
            "ms_per_step_min": round(tm["min"], 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic (seeded N(0,1)/sqrt(128) bf16 inputs, generated on the GPU)",
            "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "d": w.d, "dv": w.dv,
                       "layers": f"{w.layers[0]}..{w.layers[-1]}", "calls_per_step": len(lams),
                       "causal": True, "parallelism": "single GPU"},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                         "traffic": hbm_traffic("v1", w.name),
                         "kernel": "diffattn_v1_fwd = v1_pack_v + v1_prefill launches, HIP events per step",
                         "ms_per_launch": round(ms_call, 4),
                         "ms_per_launch_median": round(tm["median"] / len(lams), 4),
                         "ms_per_launch_min": round(tm["min"] / len(lams), 4),
                         "flop_per_launch": flop_call},
            "wall_s_timed": round(wall, 3),
        }
        del x, out, ws
        torch.cuda.empty_cache()

    iters = max(3, args.steps)

    def mfma_leg(key, name, f, flop, extra=None):
        warm_up(f, args.warmup)
        t = time_calls(f, iters, stream)
        rec = {"workload": name, **timing_fields(t, flop, 1e12, "TFLOP/s")}
        rec["frac_bf16_peak"] = round(rec["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
        rec["flop"] = flop
        rec.update(extra or {})
        secondary[key] = rec

    def hbm_leg(key, name, f, byts, extra=None):
        warm_up(f, args.warmup)
        t = time_calls(f, iters, stream)
        rec = {"workload": name, **timing_fields(t, byts, 1e9, "GB/s")}
        rec["frac_hbm_peak"] = round(rec["GB/s"] / PEAK_HBM_GBS, 4)
        rec["bytes"] = byts
        rec.update(extra or {})
        secondary[key] = rec

    # ------------------------------------------------------------------ secondary kernels
    if want("v2"):
        w = inp.V2_PREFILL
        log(f"[bench] {w.name}")
        x = inp.v2_inputs(w, device=dev)
        o = torch.empty((w.B, w.T, w.Hq // 2, w.d), dtype=torch.bfloat16, device=dev)
        mfma_leg("v2_prefill", w.name, lambda: da.v2_fwd(x["q"], x["k"], x["v"], x["logit"], out=o),
                 w.B * v2_flops_seq(w.T, w.Hq, w.d), {"traffic": hbm_traffic("v2", w.name)})
        del x, o
        torch.cuda.empty_cache()
        if cpu:
            secondary["v2_prefill"]["cpu_baseline"] = cpu_baseline_v2(w)
    for leg, key, w in (("varlen", "v2_varlen", inp.V2_VARLEN),
                        ("varlen_short", "v2_varlen_short", inp.V2_VARLEN_SHORT)):
        if not want(leg):
            continue
        log(f"[bench] {w.name} ({len(w.lengths)} sequences)")
        x = inp.v2_inputs(w, device=dev)
        N = sum(w.lengths)
        o = torch.empty((N, w.Hq // 2, w.d), dtype=torch.bfloat16, device=dev)
        mx = max(w.lengths)
        f = lambda: da.v2_fwd(x["q"], x["k"], x["v"], x["logit"], cu_seqlens=x["cu_seqlens"],
                              max_seqlen=mx, out=o)
        extra = {"nseq": len(w.lengths), "traffic": hbm_traffic(leg, w.name)}
        if len(w.lengths) <= 16:
            extra["lengths"] = list(w.lengths)
        flop = sum(v2_flops_seq(n, w.Hq, w.d) for n in w.lengths)
        # bytes the call must move: q, k, v and the logits in, out back
        byts = float(N * (w.Hq * w.d + 2 * w.Hkv * w.d) * 2 + N * (w.Hq // 2) * 4
                     + N * (w.Hq // 2) * w.d * 2)
        if max(w.lengths) <= 256:
            # short sequences: a few FLOP per byte, so the HBM roofline bounds it
            hbm_leg(key, w.name, f, byts, {**extra, "flop": flop, "bound": "hbm"})
            secondary[key]["TFLOP/s"] = round(flop / (secondary[key]["ms"] * 1e-3) / 1e12, 2)
        else:
            mfma_leg(key, w.name, f, flop, {**extra, "bytes": byts})
        del x, o
        torch.cuda.empty_cache()
        if cpu and leg == "varlen":
            secondary[key]["cpu_baseline"] = cpu_baseline_varlen(w)
    for leg, key, w in (("decode", "v2_decode", inp.V2_DECODE),
                        ("decode_b1", "v2_decode_b1", inp.V2_DECODE_B1)):
        if not want(leg):
            continue
        log(f"[bench] {w.name}")
        x = inp.decode_inputs(w, device=dev)
        o = torch.empty((w.B, w.Hq // 2, w.d), dtype=torch.bfloat16, device=dev)
        wsd = torch.empty(da.v2_decode_workspace_bytes(w.B, w.S, w.Hq, w.Hkv, w.d),
                          dtype=torch.uint8, device=dev)
        f = lambda: da.v2_decode(x["q"], x["k_cache"], x["v_cache"], x["logit"], out=o,
                                 workspace=wsd)
        hbm_leg(key, w.name, f, decode_bytes(w.B, w.S, w.Hkv, w.d),
                {"traffic": hbm_traffic(leg, w.name)})
        del x, o, wsd
        torch.cuda.empty_cache()
        if cpu and leg == "decode":
            secondary[key]["cpu_baseline"] = cpu_baseline_decode(w)
    if want("gda"):
        # grouped variant, 3 signal heads per noise head: the algorithmic count
        # attends each of the Hq query heads once, as the kernel does at this
        # ratio (blocks of 4 heads share their noise head on chip)
        w = inp.GDA_PREFILL_R3
        log(f"[bench] {w.name}")
        x = inp.v2_inputs(w, device=dev)
        o = torch.empty((w.B, w.T, w.n_out, w.d), dtype=torch.bfloat16, device=dev)
        mfma_leg("gda_prefill", w.name,
                 lambda: da.gda_fwd(x["q"], x["k"], x["v"], x["logit"], w.ratio, out=o),
                 w.B * v2_flops_seq(w.T, w.Hq, w.d),
                 {"ratio": w.ratio, "traffic": hbm_traffic("gda", w.name)})
        del x, o
        torch.cuda.empty_cache()
    if want("gda_dec"):
        w = inp.GDA_DECODE_R3
        log(f"[bench] {w.name}")
        x = inp.decode_inputs(w, device=dev)
        o = torch.empty((w.B, w.n_out, w.d), dtype=torch.bfloat16, device=dev)
        wsd = torch.empty(da.gda_decode_workspace_bytes(w.B, w.S, w.Hq, w.Hkv, w.d, w.ratio),
                          dtype=torch.uint8, device=dev)
        f = lambda: da.gda_decode(x["q"], x["k_cache"], x["v_cache"], x["logit"], w.ratio, out=o,
                                  workspace=wsd)
        hbm_leg("gda_decode", w.name, f, decode_bytes(w.B, w.S, w.Hkv, w.d),
                {"ratio": w.ratio, "traffic": hbm_traffic("gda_dec", w.name)})
        del x, o, wsd
        torch.cuda.empty_cache()
    if want("v1dec"):
        w = inp.V1_DECODE
        log(f"[bench] {w.name}")
        x = inp.v1_decode_inputs(w, device=dev)
        o = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device=dev)
        wsd = torch.empty(da.v1_decode_workspace_bytes(w.B, w.S, w.H, w.d, w.dv),
                          dtype=torch.uint8, device=dev)
        li = da.lambda_init(w.layer)
        f = lambda: da.v1_decode(x["q1"], x["q2"], x["k1_cache"], x["k2_cache"], x["v_cache"],
                                 li, li, w.eps, out=o, workspace=wsd)
        hbm_leg("v1_decode", w.name, f, 2.0 * w.B * w.S * w.H * (2 * w.d + w.dv),
                {"traffic": hbm_traffic("v1dec", w.name)})
        del x, o, wsd
        torch.cuda.empty_cache()
    if want("bwd"):
        # V2 backward on the prefill workload: the dQ (with the row values) and dK/dV
        # kernels of one diffattn_v2_bwd call; the training forward that
        # produces o_heads / lse runs once, outside the timed region
        w = inp.V2_PREFILL
        name = w.name.replace("v2_prefill", "v2_backward")
        log(f"[bench] {name}")
        x = inp.v2_inputs(w, device=dev)
        dout = inp.v2_dout(w, device=dev)
        _, oh, lse = da.v2_fwd_train(x["q"], x["k"], x["v"], x["logit"])
        wsb = torch.empty(da.v2_bwd_workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.d),
                          dtype=torch.uint8, device=dev)
        f = lambda: da.v2_bwd(x["q"], x["k"], x["v"], x["logit"], oh, lse, dout, workspace=wsb)
        mfma_leg("v2_backward", name, f, w.B * v2_bwd_flops_seq(w.T, w.Hq, w.d),
                 {"traffic": hbm_traffic("bwd", name)})
        del x, dout, oh, lse, wsb
        torch.cuda.empty_cache()
    if want("vbwd"):
        # V2 backward of the packed prefill workload (65536 tokens, 8 sequences)
        w = inp.V2_VARLEN
        name = w.name.replace("v2_varlen", "v2_varlen_backward")
        log(f"[bench] {name}")
        x = inp.v2_inputs(w, device=dev)
        dout = inp.v2_varlen_dout(w, device=dev)
        mx = max(w.lengths)
        _, oh, lse = da.v2_varlen_fwd_train(x["q"], x["k"], x["v"], x["logit"], x["cu_seqlens"], mx)
        N = sum(w.lengths)
        wsb = torch.empty(da._lib.load().diffattn_v2_varlen_bwd_workspace_bytes(
            N, len(w.lengths), w.Hq, w.Hkv, w.d), dtype=torch.uint8, device=dev)
        f = lambda: da.v2_varlen_bwd(x["q"], x["k"], x["v"], x["logit"], x["cu_seqlens"], oh, lse,
                                     dout, workspace=wsb)
        mfma_leg("v2_varlen_backward", name, f,
                 sum(v2_bwd_flops_seq(n, w.Hq, w.d) for n in w.lengths),
                 {"traffic": hbm_traffic("vbwd", name)})
        del x, dout, oh, lse, wsb
        torch.cuda.empty_cache()
    if want("v1bwd"):
        # V1 backward on the headline workload (one layer's lambda): the
        # preprocessing, reduction, dQ and dK/dV kernels of one
        # diffattn_v1_bwd call; the training forward runs once, untimed
        w = inp.V1_BF16
        name = w.name.replace("v1_bf16", "v1_backward_bf16")
        log(f"[bench] {name}")
        x = inp.v1_inputs(w, device=dev)
        dy = inp.v1_dy(w, device=dev)
        li = da.lambda_init(14)
        _, o1, o2, lse = da.v1_fwd_train(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], li, li,
                                         w.eps)
        wsb = torch.empty(da.v1_bwd_workspace_bytes(w.B, w.T, w.H, w.d, w.dv),
                          dtype=torch.uint8, device=dev)
        f = lambda: da.v1_bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], o1, o2, lse, dy, li,
                              li, w.eps, workspace=wsb)
        mfma_leg("v1_backward", name, f, v1_bwd_flops(w.B, w.T, w.H, w.d, w.dv),
                 {"traffic": hbm_traffic("v1bwd", name)})
        del x, dy, o1, o2, lse, wsb
        torch.cuda.empty_cache()
    if want("lproj") or want("proj"):
        w = inp.V2_PROJ
        log(f"[bench] {w.name}")
        x = inp.proj_inputs(w, device=dev)
        if want("lproj"):
            lg = torch.empty((w.N, w.h), dtype=torch.float32, device=dev)
            name = w.name.replace("v2_proj", "v2_lambda_proj")
            hbm_leg("v2_lambda_proj", name, lambda: da.v2_lambda_proj(x["x"], x["w_lambda"], out=lg),
                    2.0 * w.N * w.d_model + 2.0 * w.h * w.d_model + 4.0 * w.N * w.h,
                    {"traffic": hbm_traffic("lproj", name)})
            del lg
        if want("proj"):
            y = torch.empty((w.N, w.d_model), dtype=torch.bfloat16, device=dev)
            name = w.name.replace("v2_proj", "out_proj")
            mfma_leg("out_proj", name, lambda: da.out_proj(x["attn_out"], x["w_o"], out=y),
                     2.0 * w.N * w.d_model * w.h * w.d, {"traffic": hbm_traffic("proj", name)})
            del y
        del x
        torch.cuda.empty_cache()
    if secondary:
        result["secondary"] = secondary

    # ------------------------------------------------------------------ CPU oracle baseline
    if cpu and want("v1"):
        result["cpu_baseline"] = cpu_baseline()

    if "metric" not in result:
        result = {"metric": "partial run (--only)", "secondary": secondary}
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# CPU baselines: the fp64 oracle, as it stands, on bounded samples of the
# workloads (input generation outside the timed region).  ``cores`` is the
# host CPUs this process may run on; ``blas_threads`` the BLAS pool size.
# ---------------------------------------------------------------------------

def _host_threads():
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info

        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:
        blas = None
    return cores, blas


def _baseline(value, unit, spent, sample):
    cores, blas = _host_threads()
    return {"value": value, "unit": unit, "cores": cores, "blas_threads": blas, "kind": "oracle",
            "seconds": round(spent, 2), "sample": sample}


def cpu_baseline(min_s: float = 10.0, max_slices: int = 48) -> dict:
    """Time the fp64 oracle on (batch, head) slices of the headline workload.

    Slices of one layer call (layer 1, all 4096 rows) are processed in order
    until at least ``min_s`` seconds of oracle time have accumulated (or all 48
    are done).  The rate is the algorithmic FLOP of the processed slices over
    the accumulated oracle time.
    """
    import oracle
    from differential_softmax_attention_diffattn_amd import inputs as inp

    w = inp.V1_BF16
    lam = oracle.lambda_init(1)
    done = 0
    flop = 0.0
    spent = 0.0
    for b in range(w.B):
        if done >= max_slices or spent > min_s:
            break
        x = inp.v1_inputs(w.with_shape(B=1, seeds=tuple(s + 1000 * b for s in w.seeds)))
        for h in range(w.H):
            sl = [x[k][:, :, h:h + 1] for k in ("q1", "k1", "q2", "k2", "v")]
            t0 = time.perf_counter()
            oracle.v1_forward(*sl, lam, lam, w.eps)
            spent += time.perf_counter() - t0
            done += 1
            flop += v1_flops(1, w.T, 1, w.d, w.dv)
            if done >= max_slices or spent > min_s:
                break
    return _baseline(round(flop / spent / 1e12, 6), "TFLOP/s", spent,
                     f"{done} of 48 (batch, head) slices of one {w.name} layer call "
                     f"(layer 1, all 4096 rows), fp64 numpy oracle")


def cpu_baseline_v2(w, min_s: float = 5.0) -> dict:
    """The oracle on query-head pairs of the V2 prefill workload's first sequence
    (all 8192 rows each), until ``min_s`` seconds have accumulated."""
    import oracle
    from differential_softmax_attention_diffattn_amd import inputs as inp

    x = inp.v2_inputs(w.with_shape(B=1))
    g = w.Hq // w.Hkv
    spent, flop, pairs = 0.0, 0.0, 0
    for p in range(w.Hq // 2):
        kv = (2 * p) // g
        sl = (x["q"][0][:, 2 * p:2 * p + 2], x["k"][0][:, kv:kv + 1], x["v"][0][:, kv:kv + 1],
              x["logit"][0][:, p:p + 1])
        t0 = time.perf_counter()
        oracle.v2_sequence(*sl)
        spent += time.perf_counter() - t0
        flop += v2_flops_seq(w.T, 2, w.d)
        pairs += 1
        if spent > min_s:
            break
    return _baseline(round(flop / spent / 1e12, 6), "TFLOP/s", spent,
                     f"{pairs} of {w.Hq // 2 * w.B} (sequence, head pair) slices of {w.name} "
                     f"(all {w.T} rows), fp64 numpy oracle")


def cpu_baseline_varlen(w, min_s: float = 5.0) -> dict:
    """The oracle on head pairs of one mid-length sequence of the packed workload."""
    import oracle
    from differential_softmax_attention_diffattn_amd import inputs as inp

    x = inp.v2_inputs(w)
    cu = [int(c) for c in x["cu_seqlens"].tolist()]
    s = sorted(range(len(w.lengths)), key=lambda i: w.lengths[i])[len(w.lengths) // 2]
    a, e = cu[s], cu[s + 1]
    g = w.Hq // w.Hkv
    spent, flop, pairs = 0.0, 0.0, 0
    for p in range(w.Hq // 2):
        kv = (2 * p) // g
        sl = (x["q"][a:e, 2 * p:2 * p + 2], x["k"][a:e, kv:kv + 1], x["v"][a:e, kv:kv + 1],
              x["logit"][a:e, p:p + 1])
        t0 = time.perf_counter()
        oracle.v2_sequence(*sl)
        spent += time.perf_counter() - t0
        flop += v2_flops_seq(e - a, 2, w.d)
        pairs += 1
        if spent > min_s:
            break
    return _baseline(round(flop / spent / 1e12, 6), "TFLOP/s", spent,
                     f"{pairs} head pairs of sequence {s} ({e - a} tokens) of {w.name}, "
                     f"fp64 numpy oracle")


def cpu_baseline_decode(w, min_s: float = 5.0) -> dict:
    """The oracle on batch entries of the decode workload (each: every query head
    over its full 32768-entry cache), processed one (entry) at a time."""
    import oracle
    from differential_softmax_attention_diffattn_amd import inputs as inp

    small = inp.decode_small_inputs(w)
    spent, byts, done = 0.0, 0.0, 0
    for b in range(w.B):
        kc = inp.decode_cache_slice(w, b, "k")[None]
        vc = inp.decode_cache_slice(w, b, "v")[None]
        t0 = time.perf_counter()
        oracle.v2_decode(small["q"], kc, vc, small["logit"], batch=[b])
        spent += time.perf_counter() - t0
        byts += decode_bytes(1, w.S, w.Hkv, w.d)
        done += 1
        if spent > min_s:
            break
    return _baseline(round(byts / spent / 1e9, 4), "GB/s", spent,
                     f"{done} of {w.B} batch entries of {w.name} (all {w.S} cached positions, "
                     f"every head), fp64 numpy oracle")


if __name__ == "__main__":
    main()
