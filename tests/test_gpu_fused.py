"""The single-launch layer (w8a8_moe_forward_fused, decode-sized batches)
against the oracle, with the INT8 path's bar (check_moe), and against the
multi-launch layer on the same inputs (FP8 codes).

The launch keeps its per-row-block tables in LDS, so the gate-up GEMM's raw
accumulators are not captured; check_moe receives accumulators recomputed on
the host from the GPU's own codes and routing, and the GPU's gate-up GEMM is
held to bit equality through h."""
import numpy as np
import pytest
import torch

import synth
from _parity import Y_TOL, rel_metric, to_np
from test_gpu_parity import _say, _weights, check_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    import w8a8_quantized_moe_amd as w8
    return w8


def _gpu_moe_fused(w8, inp, wts, codes):
    T, H, E, k, I = inp["T"], inp["H"], inp["E"], inp["k"], inp["I"]
    lay = w8.moe_workspace_layout(T, H, E, k, I)
    ws = torch.empty((max(lay["total_bytes"], 256),), dtype=torch.uint8, device="cuda")
    y = w8.moe_forward_fused(inp["x"], wts, k, workspace=ws)
    torch.cuda.synchronize()
    g = {n: to_np(v) for n, v in w8.workspace_views(ws, T, H, E, k, I).items()}
    g["y"] = to_np(y)
    if wts.code == w8.CODE_INT8:
        xq = g["x_q"].astype(np.int64)
        wg = to_np(codes["w_gu"]).astype(np.int64)
        ids = g["topk_ids"].reshape(-1)

        def acc_rows(rows):
            a = g["sorted_assign"][np.asarray(rows)]
            return np.stack([wg[ids[ai]] @ xq[ai // k] for ai in a]).astype(np.int32)
        g["acc_gu_rows"] = acc_rows
    return g


CASES = [
    dict(T=16, H=128, E=8, k=2, I=256),
    dict(T=1, H=128, E=8, k=2, I=128),
    dict(T=37, H=384, E=5, k=3, I=384),
    dict(T=64, H=256, E=256, k=8, I=128),
    dict(T=50, H=512, E=3, k=1, I=640),
    dict(T=64, H=256, E=64, k=2, I=256, bias="zipf"),
]


@pytest.mark.parametrize("case", CASES)
def test_fused_layer_matches_oracle(w8, case):
    over = dict(n_outlier=2, outlier_scale=20.0, bf16_x=False, bias="zero", weights="int8")
    over.update(case)
    inp = synth.moe_inputs("fused", device="cuda", **over)
    check_moe(w8, inp, run=_gpu_moe_fused)


def test_fused_decode_layer_matches_oracle(w8):
    inp = synth.moe_inputs("decode", device="cuda")
    check_moe(w8, inp, run=_gpu_moe_fused)


def test_fused_layer_with_scale_options(w8):
    inp = synth.moe_inputs("fused_opts", device="cuda", T=24, H=256, E=16, k=4, I=256, n_outlier=2,
                           outlier_scale=20.0, bf16_x=False, bias="zero", weights="fp32")
    x = to_np(inp["x"])
    m = (1.0 / np.sqrt(np.abs(x).max(axis=0) + 1e-3)).astype(np.float32)  # flattens outlier columns
    m *= np.random.default_rng(5).uniform(0.9, 1.1, 256).astype(np.float32)
    clip = float(np.quantile(np.abs(x * m).max(axis=1), 0.5))  # half of the tokens are clipped
    check_moe(w8, inp, qopts=dict(x_smooth=m, x_scale_mode="clipped", x_clip=clip), run=_gpu_moe_fused)


@pytest.mark.parametrize("code", ["fp8", "fp8_fast"])
def test_fused_fp8_layer_matches_the_multi_launch_layer(w8, code):
    """E4M3 codes: the same intermediates as the multi-launch layer.  Codes
    of x exact; on rows routed to the same expert h, h_q and s_h bit for bit
    (A = 192 <= 4E, so both layers run the same register-fed GEMM items and
    sum the exact products in the same fp32 order; the tiled GEMM's 32x32
    blocks sum them in another); y within the 1e-3 bar (the logits, and so
    the routing weights, differ within the fp32 router's error)."""
    _say(f"fused FP8 layer ({code})")
    inp = synth.moe_inputs("fused_fp8", device="cuda", T=48, H=256, E=64, k=4, I=256, n_outlier=2,
                           outlier_scale=20.0, bf16_x=False, bias="zero", weights="fp8")
    T, H, E, k, I = inp["T"], inp["H"], inp["E"], inp["k"], inp["I"]
    wts = w8.MoEWeights.from_int8(inp["wr"], inp["b"], inp["w_gu"], inp["s_gu"], inp["w_d"], inp["s_d"],
                                  fp8_fast=code == "fp8_fast")
    lay = w8.moe_workspace_layout(T, H, E, k, I)
    ws_m = torch.empty((lay["total_bytes"],), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty_like(ws_m)
    y_m = w8.moe_forward(inp["x"], wts, k, workspace=ws_m)
    y_f = w8.moe_forward_fused(inp["x"], wts, k, workspace=ws_f)
    torch.cuda.synchronize()
    m = {n: to_np(v) for n, v in w8.workspace_views(ws_m, T, H, E, k, I).items()}
    f = {n: to_np(v) for n, v in w8.workspace_views(ws_f, T, H, E, k, I).items()}
    assert np.array_equal(m["x_q"], f["x_q"]) and np.array_equal(m["x_scale"], f["x_scale"])
    same = np.all(m["topk_ids"] == f["topk_ids"], axis=1)
    assert same.mean() > 0.9
    inv_m = np.empty(T * k, np.int64)
    inv_f = np.empty(T * k, np.int64)
    inv_m[m["sorted_assign"]] = np.arange(T * k)
    inv_f[f["sorted_assign"]] = np.arange(T * k)
    a = (np.where(same)[0][:, None] * k + np.arange(k)[None, :]).reshape(-1)
    for n in ("h", "h_q", "h_scale"):
        assert np.array_equal(m[n][inv_m[a]], f[n][inv_f[a]]), n
    el, mx = rel_metric(to_np(y_f)[same], to_np(y_m)[same])
    assert el <= Y_TOL and mx <= Y_TOL, (el, mx)


def test_fused_layer_is_deterministic(w8):
    inp = synth.moe_inputs("decode", device="cuda")
    wts, codes = _weights(w8, inp)
    a = _gpu_moe_fused(w8, inp, wts, codes)
    b = _gpu_moe_fused(w8, inp, wts, codes)
    for n in a:
        if not callable(a[n]):
            assert np.array_equal(a[n], b[n]), n
