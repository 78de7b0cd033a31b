"""The allocation-free entry point (w8a8_moe_forward_static) against the
workspace one (w8a8_moe_forward), through the C ABI: two calls in a row on
the library's static scratch, the second with fewer tokens than the first
(the scratch keeps the first call's contents), each bit-identical to the
workspace entry point on the same input (same kernels, same order of
operations)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def test_static_entry_point_matches_workspace_entry_point():
    import w8a8_quantized_moe_amd as w8
    inp = synth.moe_inputs("decode", device="cuda")
    T, H, E, k, I = inp["T"], inp["H"], inp["E"], inp["k"], inp["I"]
    wts = w8.MoEWeights.from_int8(inp["wr"], inp["b"], inp["w_gu"], inp["s_gu"], inp["w_d"], inp["s_d"])
    for n in (T, 23):  # the second call is smaller than the first
        print(f"static entry point: T={n} H={H} E={E} k={k} I={I}", flush=True)
        x = inp["x"][:n].contiguous()
        lay = w8.moe_workspace_layout(n, H, E, k, I)
        assert lay["total_bytes"] <= w8._lib.STATIC_WORKSPACE_BYTES
        ws = torch.empty((lay["total_bytes"],), dtype=torch.uint8, device="cuda")
        y_ref = w8.moe_forward(x, wts, k, workspace=ws)
        y = torch.full_like(x, float("nan"))
        w8.moe_forward_static(x, wts, k, y=y)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        assert np.array_equal(y.cpu().numpy(), y_ref.cpu().numpy()), f"T={n}"
    # a layer larger than the scratch is refused before any launch
    big = synth.moe_inputs("edge", device="cuda", T=4096, H=4096, E=8, k=2, I=128, n_outlier=2,
                           outlier_scale=20.0, bf16_x=False, bias="zero", weights="int8")
    assert w8.moe_workspace_layout(4096, 4096, 8, 2, 128)["total_bytes"] > w8._lib.STATIC_WORKSPACE_BYTES
    wb = w8.MoEWeights.from_int8(big["wr"], big["b"], big["w_gu"], big["s_gu"], big["w_d"], big["s_d"])
    with pytest.raises(w8.W8A8Error, match="static scratch"):
        w8.moe_forward_static(big["x"], wb, 2)
