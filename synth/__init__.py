"""Seeded synthetic inputs for the W8A8 MoE layer and the dense W8A8 GEMM.

Shared by the tests, the smoke check and the benchmark; used by both the GPU
path and the CPU oracle.  It draws random numbers only -- it holds none of the
method's arithmetic (no quantisation, routing or GEMM).  Every tensor has its
own seed derived from (seed, workload, tensor name), and is drawn with torch's
generator on the device the caller names, so the same call on the same device
type always yields the same values.  (A CPU draw and a GPU draw of the same
tensor differ; every comparison runs both sides on one draw.)

Workloads, after the five configurations of the W8A8 MoE study:

  tiny     T=16    H=128  E=8   k=2 I=256   fp32 expert weights (quantised
                                               offline by each side)
  dense    M=4096  K=8192 N=8192 dense W8A8 GEMM
  decode   T=64    H=4096 E=64  k=2 I=1536  bf16-valued x, zero router bias
  prefill  T=8192  H=4096 E=64  k=2 I=1536  Zipf-shaped router bias
  large    T=16384 H=7168 E=256 k=8 I=2048

Value recipes:
  x        N(0,1) fp32; a seeded set of outlier channels scaled by a factor
           (tiny: 2 ch x20; decode/prefill: 1% = 41 ch x20; large: 0.5% = 36
           ch x50; dense: 1% = 82 ch x30).  decode rounds x to bf16 values.
  router   W_r N(0, 0.02) fp32 [E][H]; bias zero, or for prefill
           b_e = -beta * 1.2 * ln(rank_e) with ranks a seeded permutation and
           beta calibrated so ~90% of assignments reach the 12 hottest experts
           (zipf_bias.json, written by calibrate_zipf_bias.py).
  experts  tiny: fp32 N(0, 0.02), [E][2I][H] gate/up and [E][H][I] down.
           others: int8 codes round(32 * N(0,1)) clamped to [-127, 127], with
           per-output-channel fp32 scales U(0.9, 1.1) * 0.02 * 4 / 127, i.e.
           weights of std ~0.02 already in int8 form.
  dense    A fp32 N(0,1) [M][K] with outliers; B int8 uniform in [-127, 127]
           [N][K]; per-channel scales U(0.001, 0.01).
"""
from __future__ import annotations

import hashlib
import json
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))

CONFIGS = {
    "tiny": dict(kind="moe", T=16, H=128, E=8, k=2, I=256, n_outlier=2, outlier_scale=20.0,
                 bf16_x=False, bias="zero", weights="fp32"),
    "dense": dict(kind="dense", M=4096, K=8192, N=8192, n_outlier=82, outlier_scale=30.0),
    "decode": dict(kind="moe", T=64, H=4096, E=64, k=2, I=1536, n_outlier=41, outlier_scale=20.0,
                   bf16_x=True, bias="zero", weights="int8"),
    "prefill": dict(kind="moe", T=8192, H=4096, E=64, k=2, I=1536, n_outlier=41,
                    outlier_scale=20.0, bf16_x=False, bias="zipf", weights="int8"),
    "large": dict(kind="moe", T=16384, H=7168, E=256, k=8, I=2048, n_outlier=36,
                  outlier_scale=50.0, bf16_x=False, bias="zero", weights="int8"),
}

# int8 weight recipe: codes ~ round(CODE_STD * N(0,1)), scales ~ SCALE_MID * U(0.9, 1.1)
CODE_STD = 32.0
SCALE_MID = 0.02 * 4.0 / 127.0


def _seed(seed: int, workload: str, tensor: str, part: int = 0) -> int:
    h = hashlib.sha256(f"{seed}/{workload}/{tensor}/{part}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed, workload, tensor, part=0):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, workload, tensor, part))
    return g


def zipf_beta() -> float:
    with open(os.path.join(_HERE, "zipf_bias.json")) as f:
        return float(json.load(f)["beta"])


def activations(T, H, n_outlier, outlier_scale, bf16_x, seed, workload, device):
    g = _gen(device, seed, workload, "x")
    x = torch.randn(T, H, generator=g, device=device, dtype=torch.float32)
    if n_outlier:
        go = _gen(device, seed, workload, "outlier_channels")
        ch = torch.randperm(H, generator=go, device=device)[:n_outlier]
        x[:, ch] *= outlier_scale
    if bf16_x:
        x = x.to(torch.bfloat16).to(torch.float32)
    return x.contiguous()


def router(E, H, bias_kind, seed, workload, device, beta=None):
    g = _gen(device, seed, workload, "router_w")
    wr = (torch.randn(E, H, generator=g, device=device, dtype=torch.float32) * 0.02).contiguous()
    if bias_kind == "zero":
        b = torch.zeros(E, dtype=torch.float32, device=device)
    elif bias_kind == "zipf":
        beta = zipf_beta() if beta is None else beta
        gr = _gen(device, seed, workload, "expert_rank")
        rank = torch.randperm(E, generator=gr, device=device).to(torch.float64) + 1.0
        b = (-beta * 1.2 * torch.log(rank)).to(torch.float32)
    else:
        raise ValueError(bias_kind)
    return wr, b.contiguous()


def fp32_expert_weights(E, H, I, seed, workload, device):
    g = _gen(device, seed, workload, "w_gate_up_fp32")
    w_gu = (torch.randn(E, 2 * I, H, generator=g, device=device) * 0.02).contiguous()
    g = _gen(device, seed, workload, "w_down_fp32")
    w_d = (torch.randn(E, H, I, generator=g, device=device) * 0.02).contiguous()
    return w_gu, w_d


def _int8_codes(shape, g, device):
    """round(CODE_STD * N(0,1)) clamped to [-127, 127], drawn in slabs."""
    out = torch.empty(shape, dtype=torch.int8, device=device)
    flat = out.view(shape[0], -1)
    for e in range(shape[0]):
        v = torch.randn(flat.shape[1], generator=g, device=device, dtype=torch.float32)
        flat[e] = v.mul_(CODE_STD).round_().clamp_(-127, 127).to(torch.int8)
    return out


def int8_expert_weights(E, H, I, seed, workload, device):
    g = _gen(device, seed, workload, "w_gate_up_i8")
    w_gu = _int8_codes((E, 2 * I, H), g, device)
    g = _gen(device, seed, workload, "s_gate_up")
    s_gu = (torch.rand(E, 2 * I, generator=g, device=device) * 0.2 + 0.9) * SCALE_MID
    g = _gen(device, seed, workload, "w_down_i8")
    w_d = _int8_codes((E, H, I), g, device)
    g = _gen(device, seed, workload, "s_down")
    s_d = (torch.rand(E, H, generator=g, device=device) * 0.2 + 0.9) * SCALE_MID
    return w_gu, s_gu.float().contiguous(), w_d, s_d.float().contiguous()


def fp8_expert_weights(E, H, I, seed, workload, device):
    """E4M3 codes (uint8) of weights with std ~0.02: code values ~N(0, 64),
    clipped to the E4M3 range, times per-channel scales ~U(0.9, 1.1)*0.02/64.
    The codes are random inputs; their conversion is torch's, not the method's."""
    def codes(shape, name):
        g = _gen(device, seed, workload, name)
        v = (torch.randn(shape, generator=g, device=device) * 64.0).clamp(-448.0, 448.0)
        return v.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    w_gu = codes((E, 2 * I, H), "w_gate_up_fp8")
    w_d = codes((E, H, I), "w_down_fp8")
    g = _gen(device, seed, workload, "s_gate_up")
    s_gu = (torch.rand(E, 2 * I, generator=g, device=device) * 0.2 + 0.9) * (0.02 / 64.0)
    g = _gen(device, seed, workload, "s_down")
    s_d = (torch.rand(E, H, generator=g, device=device) * 0.2 + 0.9) * (0.02 / 64.0)
    return w_gu, s_gu.float().contiguous(), w_d, s_d.float().contiguous()


def moe_inputs(workload="tiny", seed=0, device="cpu", **override):
    """Inputs of one MoE workload.  ``override`` replaces shape/recipe fields
    (T, H, E, k, I, n_outlier, outlier_scale, bf16_x, bias, weights, beta).

    Returns a dict with x, wr, b and either (w_gu_f32, w_d_f32) for fp32
    weights or (w_gu, s_gu, w_d, s_d) for int8 (or, weights="fp8", uint8 E4M3)
    codes, plus the shape."""
    cfg = dict(CONFIGS[workload]) if workload in CONFIGS else dict(CONFIGS["tiny"])
    cfg.update(override)
    assert cfg["kind"] == "moe"
    T, H, E, k, I = cfg["T"], cfg["H"], cfg["E"], cfg["k"], cfg["I"]
    out = dict(T=T, H=H, E=E, k=k, I=I, workload=workload)
    out["x"] = activations(T, H, cfg["n_outlier"], cfg["outlier_scale"], cfg["bf16_x"], seed,
                           workload, device)
    out["wr"], out["b"] = router(E, H, cfg["bias"], seed, workload, device, cfg.get("beta"))
    if cfg["weights"] == "fp32":
        out["w_gu_f32"], out["w_d_f32"] = fp32_expert_weights(E, H, I, seed, workload, device)
    elif cfg["weights"] == "fp8":
        out["w_gu"], out["s_gu"], out["w_d"], out["s_d"] = fp8_expert_weights(
            E, H, I, seed, workload, device)
    else:
        out["w_gu"], out["s_gu"], out["w_d"], out["s_d"] = int8_expert_weights(
            E, H, I, seed, workload, device)
    return out


def dense_inputs(workload="dense", seed=0, device="cpu", **override):
    cfg = dict(CONFIGS["dense"])
    cfg.update(override)
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    a = activations(M, K, cfg["n_outlier"], cfg["outlier_scale"], False, seed, workload, device)
    g = _gen(device, seed, workload, "b_i8")
    b = torch.randint(-127, 128, (N, K), generator=g, device=device, dtype=torch.int16).to(torch.int8)
    g = _gen(device, seed, workload, "s_b")
    s_b = (torch.rand(N, generator=g, device=device) * 0.009 + 0.001).float()
    return dict(M=M, K=K, N=N, a=a, b=b.contiguous(), s_b=s_b.contiguous())


def moe_flops(T, H, E, k, I):
    """int8 expert-GEMM operations of one layer pass: 2*A*(H*2I + I*H)."""
    return 6 * T * k * H * I


def zipf_top12_share(counts):
    c = sorted((int(v) for v in counts), reverse=True)
    tot = sum(c)
    return sum(c[:12]) / tot if tot else math.nan
