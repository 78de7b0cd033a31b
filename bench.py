#!/usr/bin/env python3
"""Benchmark of the W8A8 MoE expert layer on one MI355X.

One step = one whole pass of the layer (per-token quantisation, fp32 router +
top-k + permutation, grouped gate-up GEMM with the SwiGLU epilogue,
requantisation, grouped down GEMM with the weighted scatter, combine) over one
batch of seeded synthetic tokens already resident in HBM.  W untimed warm-up
steps, then exactly K timed steps between two device synchronisations.

Default workload: the large fine-grained layer (T=16384 tokens, H=7168,
E=256 experts, top-8, I=2048, ~11.3 GB of int8 expert weights), the largest
MoE configuration of the study, which fits one GPU.

Prints one JSON line: tokens/s of the whole job over the K timed steps, the
per-stage times (HIP events recorded on the layer's stream at every stage
boundary, in a separate pass of K steps before the timed ones), the roofline
of the dominant kernel (its launch time from the two events around it in
every timed step), whole-layer INT8 TOPS and algorithmic HBM GB/s, the rate
a plain 1 GiB device copy attains (measured after the timed steps), the
device's CU count and peak clock, and the CPU oracle timed on a bounded token
sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks (dense)
PEAK_INT8_OPS = 5.0e15      # int8 MFMA, ops/s
PEAK_FP8_OPS = 5.0e15       # fp8 MFMA, flop/s (the same as int8 on this chip)
PEAK_BF16_OPS = 2.5e15      # bf16 MFMA, flop/s (the exact FP8 path multiplies decoded codes here)
PEAK_FP32_MFMA = 157.3e12   # fp32 matrix, flop/s
PEAK_HBM = 8.0e12           # bytes/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles created through the HIP runtime (plumbing for timing)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, arr):
        for ev in arr:
            self.hip.hipEventDestroy(ev)


# Per-dispatch hardware counters of each stage's kernels, measured with
# rocprofv3 (FETCH_SIZE and WRITE_SIZE each in its own pass, scaled by what the
# same counters read for a plain device copy of known size; GRBM_COUNT for the
# engine clock the kernel ran at; SQ_VALU_MFMA_BUSY_CYCLES).  Valid only for
# the kernel sources they were measured on: the hash below must match the
# sources as they are now.
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = ["w8a8_quantized_moe_amd/csrc/gemm.hip", "w8a8_quantized_moe_amd/csrc/internal.h",
                  "w8a8_quantized_moe_amd/csrc/device_common.h", "w8a8_quantized_moe_amd/csrc/skinny_item.h",
                  "w8a8_quantized_moe_amd/csrc/route.hip", "w8a8_quantized_moe_amd/csrc/quant.hip",
                  "w8a8_quantized_moe_amd/csrc/combine.hip", "w8a8_quantized_moe_amd/csrc/skinny.hip",
                  "w8a8_quantized_moe_amd/csrc/abi.cpp"]
# The single-launch layer (fused.hip) has a kernel trace but no counter record,
# so its source is not part of the hash.
PEAK_CLOCK_MHZ = 2400.0  # the engine clock the published matrix peaks assume
EVENT_EVERY = 5  # timed steps per step that records the dominant stage's events


def _code_only(text):
    """Source text without comments and blank lines (a comment edit does not
    change the kernels the counters were taken on)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_sources_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def measured_counters(workload, stage, code="int8"):
    """The stage's counter record from profiles/counters.json, or None when
    there is none or the kernels changed since it was taken."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_hash():
        return None
    key = f"{workload}:{stage}" if code == "int8" else f"{workload}/{code}:{stage}"
    return rec.get("stages", {}).get(key)


def counter_fields(ent, bound, achieved, peak):
    """traffic (HBM bytes per launch), and for a matrix-bound kernel the engine
    clock it sustained, the fraction of the peak scaled to that clock, and the
    MFMA-busy fraction; None where no valid counter record exists."""
    out = {"traffic": None}
    if not ent:
        return out
    out["traffic"] = int(ent["fetch_bytes"] + ent["write_bytes"])
    clk = ent.get("clock_mhz")
    if bound == "mfma" and clk:
        out["sustained_clock_mhz"] = clk
        out["frac_at_sustained_clock"] = round(achieved / (peak * clk / PEAK_CLOCK_MHZ), 4)
        out["mfma_busy"] = ent.get("mfma_busy")
    return out


def copy_calibration(torch, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size: what FETCH_SIZE and
    WRITE_SIZE read for it converts the counters to bytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes_each_way": nbytes, "reps": reps, "ms": round(dt * 1e3, 4),
                      "gbps_read_plus_write": round(2 * nbytes / dt / 1e9, 1)}), flush=True)


def attainable_hbm(torch, nbytes=1 << 30, reps=10):
    """What a plain device copy reaches on this device (context for the
    roofline fractions, which use the published 8 TB/s): a 1 GiB copy, bytes
    read plus written, timed with events after a warm-up."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (s.elapsed_time(e) * 1e-3) / 1e9
    del src, dst
    return {"copy_GBps": round(gbps, 1), "frac_of_peak": round(gbps * 1e9 / PEAK_HBM, 4),
            "method": f"torch copy_ of 1 GiB fp32, {reps} reps, read + write bytes"}


def device_info(torch):
    """Compute units and the peak engine clock (rocminfo), with the INT8 matrix
    peak they imply (8192 int8 ops per CU per clock), beside the published one."""
    info = {"cus": torch.cuda.get_device_properties(0).multi_processor_count, "max_sclk_mhz": None}
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        for blk in txt.split("Agent ")[1:]:
            if "gfx950" in blk:
                m = re.search(r"Max Clock Freq\. \(MHz\):\s*(\d+)", blk)
                info["max_sclk_mhz"] = int(m.group(1)) if m else None
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if info["max_sclk_mhz"]:
        info["int8_peak_at_max_clock_tops"] = round(8192 * info["cus"] * info["max_sclk_mhz"] / 1e6, 1)
    return info


def stage_work(T, H, E, k, I, touched, code="int8"):
    """Algorithmic work per launch of each stage: (bound, amount, unit, peak).

    The grouped GEMMs count both their int8 ops and their algorithmic bytes
    (the touched experts' weights and scales once, the activation rows each
    assignment reads, the output written); the bound is the one their
    arithmetic intensity selects against the ridge point peak_ops/peak_bytes.
    """
    A = T * k
    gu_ops, dn_ops = 2 * A * H * 2 * I, 2 * A * I * H
    gu_bytes = touched * (2 * I * H + 8 * I) + A * H + 4 * T + 4 * A * I
    dn_bytes = touched * (H * I + 4 * H) + A * I + 8 * A + 4 * A * H
    peak_mma = {"int8": PEAK_INT8_OPS, "fp8": PEAK_BF16_OPS, "fp8_fast": PEAK_FP8_OPS}[code]
    ridge = peak_mma / PEAK_HBM

    def gemm(ops, nbytes):
        if ops / nbytes >= ridge:
            return ("mfma", ops, "TOP/s" if code == "int8" else "TFLOP/s", peak_mma)
        return ("hbm", nbytes, "GB/s", PEAK_HBM)

    return {
        "quant": ("hbm", 4 * T * H + T * H + 4 * T, "GB/s", PEAK_HBM),
        "route": ("mfma", 2 * T * H * E, "TFLOP/s", PEAK_FP32_MFMA),
        "gate_up": gemm(gu_ops, gu_bytes),
        "requant": ("hbm", 4 * A * I + A * I + 4 * A, "GB/s", PEAK_HBM),
        "down": gemm(dn_ops, dn_bytes),
        "combine": ("hbm", 4 * A * H + 4 * T * H, "GB/s", PEAK_HBM),
    }


def cpu_baseline(inp, target_s, code="int8"):
    """The CPU oracle, as it stands, on the first n tokens of the same batch
    (whole layer for those tokens), n sized for about target_s seconds."""
    import numpy as np

    import oracle
    x = inp["x"].cpu().numpy()
    wr = inp["wr"].cpu().numpy()
    b = inp["b"].cpu().numpy()
    k, T = inp["k"], inp["T"]
    if "w_gu_f32" in inp:
        # fp32 weights: the oracle quantises them itself (per output channel),
        # as it does in the parity tests; nothing it runs on comes from the GPU path
        E, I2, H = inp["w_gu_f32"].shape
        quant = oracle.quantize_rows if code == "int8" else oracle.quantize_rows_fp8
        w_gu, s_gu = quant(inp["w_gu_f32"].cpu().numpy().reshape(E * I2, H))
        w_gu, s_gu = w_gu.reshape(E, I2, H), s_gu.reshape(E, I2)
        w_d, s_d = quant(inp["w_d_f32"].cpu().numpy().reshape(E * H, I2 // 2))
        w_d, s_d = w_d.reshape(E, H, I2 // 2), s_d.reshape(E, H)
    else:
        w_gu = inp["w_gu"].cpu().numpy()
        s_gu = inp["s_gu"].cpu().numpy()
        w_d = inp["w_d"].cpu().numpy()
        s_d = inp["s_d"].cpu().numpy()

    def run(n):
        t0 = time.perf_counter()
        oracle.moe_forward(x, wr, b, w_gu, s_gu, w_d, s_d, k, route_tokens=np.arange(n),
                           code="int8" if code == "int8" else "fp8")
        return time.perf_counter() - t0

    probe_n = min(8, T)
    t_probe = run(probe_n)
    n = int(max(probe_n, min(T, target_s / max(t_probe / probe_n, 1e-9))))
    t = run(n) if n != probe_n else t_probe
    return dict(value=n / t, unit="tokens/s", cores=oracle.max_threads(), kind="oracle",
                sample=f"first {n} of {T} tokens of the same batch, whole layer for them "
                       f"(quant, fp64 router, softmax/top-k, permute, expert FFN, combine); "
                       f"{t:.1f} s", seconds=t, tokens=n)


def bench_dense(args, torch, synth, w8):
    """The dense W8A8 GEMM workload (M=4096, K=8192, N=8192): one step = the
    per-token quantisation of A plus the int8 GEMM with the scale epilogue."""
    log("[bench] generating the dense GEMM workload on the GPU")
    inp = synth.dense_inputs(device="cuda")
    M, K, N = inp["M"], inp["K"], inp["N"]
    bp = w8.pack_weights(inp["b"])
    a_q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s_a = torch.empty((M,), dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    hip = HipEvents()
    events = [hip.create(3) for _ in range(args.steps)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hip.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def step(ev=None):
        if ev is not None:
            hip.hip.hipEventRecord(ev[0], stream)
        w8.quantize_rows(inp["a"], a_q, s_a)
        if ev is not None:
            hip.hip.hipEventRecord(ev[1], stream)
        w8.gemm(a_q, s_a, bp, inp["s_b"], N, K, out=out)
        if ev is not None:
            hip.hip.hipEventRecord(ev[2], stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sampled = [i for i in range(args.steps) if i % EVENT_EVERY == 0]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i] if i % EVENT_EVERY == 0 else None)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    q_ms = sum(hip.elapsed_ms(events[i][0], events[i][1]) for i in sampled) / len(sampled)
    g_ms = sum(hip.elapsed_ms(events[i][1], events[i][2]) for i in sampled) / len(sampled)
    ops = 2 * M * N * K
    q_bytes = 4 * M * K + M * K + 4 * M
    out_line = {
        "metric": "dense W8A8 GEMM INT8 TOPS (per-token quant + GEMM with scale epilogue)",
        "value": round(ops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded)",
        "config": {"workload": f"dense W8A8 GEMM M={M} K={K} N={N}", "M": M, "K": K, "N": N},
        "stage_ms": {"quant": round(q_ms, 4), "gemm": round(g_ms, 4)},
        "roofline": dict(kernel="gemm", bound="mfma", achieved=round(ops / (g_ms * 1e-3) / 1e12, 2),
                         peak=PEAK_INT8_OPS / 1e12, unit="TOP/s",
                         frac=round(ops / (g_ms * 1e-3) / PEAK_INT8_OPS, 4),
                         work_per_launch=ops,
                         **counter_fields(measured_counters("dense", "gemm"), "mfma",
                                          ops / (g_ms * 1e-3), PEAK_INT8_OPS)),
        "quant_roofline": dict(bound="hbm", achieved=round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
                               peak=PEAK_HBM / 1e9, unit="GB/s",
                               frac=round(q_bytes / (q_ms * 1e-3) / PEAK_HBM, 4)),
    }
    for e in events:
        hip.destroy(e)
    if not args.kernels_only:
        out_line["attainable_hbm"] = attainable_hbm(torch)
        out_line["device"] = device_info(torch)
    print(json.dumps(out_line), flush=True)


def time_stages(args, torch, w8, inp, wts, k, y, ws, hip, events, stages):
    """The multi-launch layer: per-stage times from a separate pass with an
    event at every stage boundary, then K timed steps recording the dominant
    stage's two events in every EVENT_EVERY-th step.  Returns (stage_ms,
    event_step_ms, dominant stage, ms per step, dominant stage's ms)."""
    # Stage breakdown: a separate pass of K steps with an event at every stage
    # boundary (each recorded event costs a few microseconds on the stream, a
    # tenth of a decode step over the seven boundaries, so the timed pass
    # below records only the two around the dominant stage).
    log(f"[bench] stage breakdown over {args.steps} steps")
    for i in range(args.steps):
        w8.moe_forward(inp["x"], wts, k, y=y, workspace=ws, events=events[i])
    torch.cuda.synchronize()
    stage_ms = {s: 0.0 for s in stages}
    event_step_ms = 0.0
    for ev in events:
        for j, s in enumerate(stages):
            stage_ms[s] += hip.elapsed_ms(ev[j], ev[j + 1]) / args.steps
        event_step_ms += hip.elapsed_ms(ev[0], ev[len(stages)]) / args.steps
    dom = max(stages, key=lambda s: stage_ms[s])
    jd = stages.index(dom)
    # the timed pass: events only at the dominant stage's two boundaries, and
    # only in every EVENT_EVERY-th step (each recorded event costs ~3 us on the
    # stream: recorded in every step, the two would add 3% to a decode step)
    timed_ev = []
    for ev in events:
        arr = (ctypes.c_void_p * (len(stages) + 1))()
        arr[jd], arr[jd + 1] = ev[jd], ev[jd + 1]
        timed_ev.append(arr)
    sampled = [i for i in range(args.steps) if i % EVENT_EVERY == 0]

    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        w8.moe_forward(inp["x"], wts, k, y=y, workspace=ws,
                       events=timed_ev[i] if i % EVENT_EVERY == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dom_ms = sum(hip.elapsed_ms(events[i][jd], events[i][jd + 1]) for i in sampled) / len(sampled)
    for ev in events:
        hip.destroy(ev)

    return stage_ms, event_step_ms, dom, ms_per_step, dom_ms


def time_fused(args, torch, w8, inp, wts, k, y, ws, hip, events):
    """The single-launch layer: K timed steps; every EVENT_EVERY-th records two
    events around the launch on the layer's stream (torch's current stream).
    The layer is one kernel, so it is its own dominant stage."""
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hip.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    sampled = [i for i in range(args.steps) if i % EVENT_EVERY == 0]
    log(f"[bench] timing {args.steps} steps (single launch)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % EVENT_EVERY == 0:
            hip.hip.hipEventRecord(events[i][0], stream)
        w8.moe_forward_fused(inp["x"], wts, k, y=y, workspace=ws)
        if i % EVENT_EVERY == 0:
            hip.hip.hipEventRecord(events[i][1], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dom_ms = sum(hip.elapsed_ms(events[i][0], events[i][1]) for i in sampled) / len(sampled)
    for ev in events:
        hip.destroy(ev)
    return {"fused": round(dom_ms, 4)}, dom_ms, "fused", ms_per_step, dom_ms


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large",
                    choices=["large", "prefill", "decode", "tiny", "dense"])
    ap.add_argument("--code", default="int8", choices=["int8", "fp8", "fp8_fast"],
                    help="code type of the expert weights and activations (fp8: E4M3 codes, exact "
                         "products summed in fp32 on the bf16 matrix cores; fp8_fast: E4M3 codes on "
                         "the FP8 matrix cores)")
    ap.add_argument("--weights", default="codes", choices=["codes", "fp32"],
                    help="expert weights of the decode, prefill and large layers: codes (int8 or E4M3 "
                         "codes drawn directly, with per-channel scales) or fp32 (fp32 N(0, 0.02) "
                         "weights quantised per output channel by the library's offline quantiser)")
    ap.add_argument("--fused", action="store_true",
                    help="run the layer as one persistent launch (w8a8_moe_forward_fused; T <= 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels-only", action="store_true",
                    help="time the layer only: no device-copy rate, no rocminfo query, no CPU "
                         "baseline (for runs under a counter profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for the traffic field)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only: the layer runs on a single "
                          "MI355X (no collectives); run with --gpus 1"}), flush=True)
        sys.exit(2)

    import torch

    import synth
    import w8a8_quantized_moe_amd as w8

    torch.cuda.set_device(0)
    if args.copy_calibration:
        return copy_calibration(torch)
    if args.workload == "dense":
        return bench_dense(args, torch, synth, w8)
    log(f"[bench] generating workload '{args.workload}' on the GPU")
    over = {} if args.code == "int8" else {"weights": "fp8"}
    if args.weights == "fp32":
        over = {"weights": "fp32"}
    inp = synth.moe_inputs(args.workload, device="cuda", **over)
    T, H, E, k, I = inp["T"], inp["H"], inp["E"], inp["k"], inp["I"]
    A = T * k
    if "w_gu_f32" in inp:
        code = {"int8": w8.CODE_INT8, "fp8": w8.CODE_FP8, "fp8_fast": w8.CODE_FP8_FAST}[args.code]
        wts = w8.MoEWeights.from_fp32(inp["wr"], inp["b"], inp["w_gu_f32"], inp["w_d_f32"], code=code)
    else:
        wts = w8.MoEWeights.from_int8(inp["wr"], inp["b"], inp["w_gu"], inp["s_gu"], inp["w_d"],
                                      inp["s_d"], fp8_fast=args.code == "fp8_fast")
    lay = w8.moe_workspace_layout(T, H, E, k, I)
    ws = torch.empty((lay["total_bytes"],), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(inp["x"])
    torch.cuda.synchronize()

    stages = w8._lib.MOE_STAGES
    hip = HipEvents()
    events = [hip.create(len(stages) + 1) for _ in range(args.steps)]

    log(f"[bench] warmup {args.warmup} steps")
    if args.fused and T > w8._lib.FUSED_MAX_T:
        raise SystemExit(f"--fused runs layers of at most {w8._lib.FUSED_MAX_T} tokens (this one has {T})")
    forward = w8.moe_forward_fused if args.fused else w8.moe_forward
    for _ in range(args.warmup):
        forward(inp["x"], wts, k, y=y, workspace=ws)
    torch.cuda.synchronize()

    if args.fused:
        stage_ms, event_step_ms, dom, ms_per_step, dom_ms = time_fused(args, torch, w8, inp, wts, k, y, ws, hip,
                                                                      events)
    else:
        stage_ms, event_step_ms, dom, ms_per_step, dom_ms = time_stages(args, torch, w8, inp, wts, k, y, ws, hip,
                                                                       events, stages)

    counts = w8.workspace_views(ws, T, H, E, k, I)["expert_counts"].cpu()
    touched = int((counts > 0).sum())
    work = stage_work(T, H, E, k, I, touched, args.code)
    alg_bytes = 8 * T * H + 4 * H * E + 4 * E + touched * (3 * H * I + 4 * (2 * I + H))
    work["fused"] = ("hbm", alg_bytes, "GB/s", PEAK_HBM)
    bound, amount, unit, peak = work[dom]
    scale = 1e9 if unit == "GB/s" else 1e12
    achieved = amount / (dom_ms * 1e-3)
    roofline = dict(kernel=dom, bound=bound, achieved=round(achieved / scale, 2),
                    peak=peak / scale, unit=unit, frac=round(achieved / peak, 4), work_per_launch=amount,
                    **counter_fields(measured_counters(args.workload, dom, args.code), bound, achieved, peak))

    step_s = ms_per_step * 1e-3
    int8_ops = 6 * A * H * I

    out = {
        "metric": "MoE-layer tokens/s; INT8 TOPS & HBM GB/s as % of MI355X roofline",
        "value": round(T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if args.code == "int8" else "fp8_e4m3",
        "data": (f"synthetic (seeded; random {'int8' if args.code == 'int8' else 'FP8 E4M3'} expert "
                 "weights of the layer's shape)") if "w_gu_f32" not in inp else
                f"synthetic (seeded; fp32 N(0, 0.02) expert weights of the layer's shape, quantised per "
                f"output channel to {'int8' if args.code == 'int8' else 'FP8 E4M3'} codes)",
        "config": {"workload": f"{args.workload} MoE layer T={T} H={H} E={E} top-{k} I={I}"
                               + {"int8": "", "fp8": ", FP8 E4M3 codes (exact products, fp32 sums)",
                                  "fp8_fast": ", FP8 E4M3 codes on the FP8 matrix cores"}[args.code],
                   "T": T, "H": H, "E": E, "top_k": k, "I": I, "code": args.code,
                   "weights": "fp32 quantised" if "w_gu_f32" in inp else "codes",
                   "launch": "one persistent launch" if args.fused else "one launch per stage",
                   "parallelism": "none (1 GPU)"},
        f"{args.code}_tops": round(int8_ops / step_s / 1e12, 2),
        f"{args.code}_frac_of_peak": round(int8_ops / step_s / work["gate_up"][3], 4)
        if work["gate_up"][0] == "mfma" else round(int8_ops / step_s / PEAK_INT8_OPS, 4),
        "alg_hbm_gbps": round(alg_bytes / step_s / 1e9, 1),
        "hbm_frac_of_peak": round(alg_bytes / step_s / PEAK_HBM, 4),
        "experts_touched": touched,
        "event_ms_per_step": round(event_step_ms, 4),
        "stage_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "roofline": roofline,
    }
    if not args.kernels_only:
        out["attainable_hbm"] = attainable_hbm(torch)
        out["device"] = device_info(torch)
    if not (args.no_cpu_baseline or args.kernels_only):
        log("[bench] timing the CPU oracle on a token sample")
        cb = cpu_baseline(inp, args.cpu_seconds, args.code)
        out["cpu_baseline"] = {kk: (round(v, 3) if isinstance(v, float) else v)
                               for kk, v in cb.items() if kk in ("value", "unit", "cores", "kind",
                                                                 "sample")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
