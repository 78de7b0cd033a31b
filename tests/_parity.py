"""Helpers of the GPU-vs-oracle parity tests (test infrastructure).

The oracle always runs on its own inputs (the seeded synthetic tensors, copied
to the host); nothing the GPU computed is ever fed into it.  Comparison rules:

* int8 codes, int32 results, indices and permutations: bit-exact.
* top-k ids: bit-exact, except tokens whose oracle (fp64) logits have a near
  tie at the selection boundary or inside the selected order -- a gap below
  max(1e-5, 2 * the largest |GPU logit - oracle logit| of that token).  Those
  are counted and excluded from the exact downstream comparisons; for every
  token the GPU ids must still be a valid top-k of the GPU's own logits.
* h: bit-exact on every row (both sides evaluate SiLU with a correctly
  rounded exponential and IEEE fp32 operations), and so are h's scales and
  codes.  The grouped GEMMs' int32 accumulators are compared exactly: the
  gate-up ones directly, the down ones through o, which must equal the
  epilogue on the oracle's accumulators (corrected for moved codes) bit for
  bit; o against the oracle's own is then within the routing weight's error.
* the combined output y = sum_j o_j: error <= 1e-3 relative to sum_j |o_j|
  and to the row maximum (sum_rel_metric); element-wise relative error is
  reported but not bounded, since it is ill-conditioned where terms cancel.
"""
from __future__ import annotations

import numpy as np
import torch

Y_TOL = 1e-3


def rel_metric(got: np.ndarray, ref: np.ndarray):
    """(element-wise relative error over elements with |ref| >= 1e-3 * row max,
    max |got - ref| / row max over all elements) -- both must be <= 1e-3."""
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    rowmax = np.abs(ref).max(axis=1, keepdims=True)
    rowmax = np.where(rowmax == 0, 1.0, rowmax)
    big = np.abs(ref) >= 1e-3 * rowmax
    err = np.abs(got - ref)
    elem = (err / np.where(big, np.abs(ref), 1.0))[big]
    return (float(elem.max()) if elem.size else 0.0), float((err / rowmax).max())


def valid_topk(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Per token: ids are distinct, ordered by descending logit (ties by
    ascending index), and every selected logit >= every unselected one, with
    ties at the boundary resolved toward lower indices."""
    T, E = logits.shape
    k = ids.shape[1]
    ok = np.ones(T, bool)
    for t in range(T):
        sel = ids[t]
        if len(set(sel.tolist())) != k or sel.min() < 0 or sel.max() >= E:
            ok[t] = False
            continue
        key = [(-float(logits[t, e]), int(e)) for e in sel]
        if key != sorted(key):
            ok[t] = False
            continue
        rest = np.setdiff1d(np.arange(E), sel)
        if rest.size:
            worst = key[-1]  # the k-th pick
            for e in rest:
                if (-float(logits[t, e]), int(e)) < worst:
                    ok[t] = False
                    break
    return ok


def near_tie_tokens(l_ora: np.ndarray, l_gpu: np.ndarray, k: int) -> np.ndarray:
    """Tokens whose oracle selection or order is within numerical noise."""
    T, E = l_ora.shape
    delta = np.abs(l_gpu.astype(np.float64) - l_ora).max(axis=1)
    thr = np.maximum(1e-5, 2.0 * delta)
    srt = -np.sort(-l_ora, axis=1)
    upto = min(k + 1, E)
    gaps = srt[:, :upto - 1] - srt[:, 1:upto]
    return (gaps < thr[:, None]).any(axis=1) if gaps.size else np.zeros(T, bool)


def sum_rel_metric(got: np.ndarray, ref: np.ndarray, terms_abs_sum: np.ndarray):
    """Error of a sum measured against the sum of its terms' magnitudes:
    max |got - ref| / sum_j |o_j| (elements whose terms are all zero must be
    exact), and max |got - ref| / row max |ref|.  Element-wise relative error
    is ill-conditioned where the k weighted expert outputs cancel."""
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    err = np.abs(got - ref)
    den = terms_abs_sum.astype(np.float64)
    if np.any(err[den == 0] != 0):
        return np.inf, np.inf
    s = float((err[den > 0] / den[den > 0]).max()) if np.any(den > 0) else 0.0
    rowmax = np.abs(ref).max(axis=1, keepdims=True)
    rowmax = np.where(rowmax == 0, 1.0, rowmax)
    return s, float((err / rowmax).max())


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def stable_sort_assign(ids: np.ndarray) -> np.ndarray:
    return np.argsort(ids.reshape(-1), kind="stable").astype(np.int32)
