"""The layer captured in a HIP graph (through torch.cuda.CUDAGraph): every
launch of w8a8_moe_forward goes onto the caller's stream, and the library
allocates nothing, synchronises nothing and issues no memset (the routing
kernels zero the GEMMs' tile counters), so the call can be captured once and
replayed.  Each replay must reproduce the eager result bit for bit, with
unrelated eager work and synchronisations between the replays."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    import w8a8_quantized_moe_amd as w8mod
    return w8mod


def _weights(w8, inp):
    if "w_gu_f32" in inp:
        return w8.MoEWeights.from_fp32(inp["wr"], inp["b"], inp["w_gu_f32"], inp["w_d_f32"])
    return w8.MoEWeights.from_int8(inp["wr"], inp["b"], inp["w_gu"], inp["s_gu"], inp["w_d"], inp["s_d"])


@pytest.mark.parametrize("workload,over", [
    ("decode", {}),                                                    # skinny GEMMs, fused routing
    ("edge", dict(T=300, H=256, E=8, k=2, I=256, n_outlier=2, outlier_scale=20.0, bf16_x=False,
                  bias="zero", weights="int8")),                        # tiled persistent GEMMs
    ("edge", dict(T=300, H=256, E=8, k=2, I=256, n_outlier=2, outlier_scale=20.0, bf16_x=False,
                  bias="zero", weights="fp8")),                         # the same with E4M3 codes
    ("edge", dict(T=2100, H=512, E=100, k=4, I=256, n_outlier=2, outlier_scale=20.0, bf16_x=False,
                  bias="zero", weights="int8")),                        # router weights split into planes
], ids=["decode", "tiled", "tiled-fp8", "router-planes"])
def test_moe_forward_graph_replays_match_eager(w8, workload, over):
    print(f"graph capture: {workload} {over}", flush=True)
    inp = synth.moe_inputs(workload, device="cuda", **over)
    T, H, E, k, I = inp["T"], inp["H"], inp["E"], inp["k"], inp["I"]
    wts = _weights(w8, inp)
    lay = w8.moe_workspace_layout(T, H, E, k, I)
    ws = torch.empty((lay["total_bytes"],), dtype=torch.uint8, device="cuda")
    x = inp["x"]
    y = torch.empty_like(x)
    y_ref = w8.moe_forward(x, wts, k, workspace=ws).clone()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w8.moe_forward(x, wts, k, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        w8.moe_forward(x, wts, k, y=y, workspace=ws)
    torch.cuda.synchronize()

    # unrelated eager work between replays, into its own buffers
    x2 = (x * 0.5).contiguous()
    ws2 = torch.empty_like(ws)
    for rep in range(4):
        y.fill_(float("nan"))
        ws.fill_(0xA5)          # stale workspace contents must not matter
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep} differs from the eager result"
        w8.moe_forward(x2, wts, k, workspace=ws2)
        torch.cuda.synchronize()
