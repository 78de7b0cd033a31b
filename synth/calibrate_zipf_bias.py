"""Calibrate the Zipf-shaped router bias of the skewed prefill workload.

The skewed workload wants a Zipf(1.2)-shaped expert popularity that sends
about 90% of assignments to the 12 hottest of 64 experts (the RTX 3090 /
Strata page, sec. 2.1, observes that 12 of 64 experts take over 90% of
routing).  A plain Zipf(1.2) law over 64 ranks gives only ~75% to the top 12,
so the shape b_e = -beta * 1.2 * ln(rank_e) is kept and beta is bisected until
the realised top-12 share of the oracle's own routing is 0.90.

Routing is computed with the CPU oracle only (fp64 logits, softmax/top-k) on
CPU-drawn inputs of the prefill shape; the result is written to
zipf_bias.json beside this file.  Run:  python -m synth.calibrate_zipf_bias
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
import synth


def main():
    cfg = synth.CONFIGS["prefill"]
    T, H, E, k = cfg["T"], cfg["H"], cfg["E"], cfg["k"]
    x = synth.activations(T, H, cfg["n_outlier"], cfg["outlier_scale"], cfg["bf16_x"], 0,
                          "prefill", "cpu").numpy()
    wr, _ = synth.router(E, H, "zero", 0, "prefill", "cpu")
    base = oracle.router_logits(x, wr.numpy(), None)

    def share(beta):
        _, b = synth.router(E, H, "zipf", 0, "prefill", "cpu", beta=beta)
        ids, _ = oracle.topk_softmax(base + b.numpy().astype(np.float64)[None, :], k)
        counts = np.bincount(ids.reshape(-1), minlength=E)
        return synth.zipf_top12_share(counts), counts

    lo, hi = 0.0, 10.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        s, _ = share(mid)
        if s < 0.90:
            lo = mid
        else:
            hi = mid
    beta = 0.5 * (lo + hi)
    s, counts = share(beta)
    out = dict(beta=beta, top12_share=s, counts_sorted=sorted(map(int, counts), reverse=True),
               experts_with_at_most_3=int((counts <= 3).sum()),
               note="beta for b_e = -beta*1.2*ln(rank_e); calibrated on CPU-drawn prefill inputs, "
                    "seed 0, with the CPU oracle's routing")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    torch.set_num_threads(os.cpu_count() or 1)
    main()
