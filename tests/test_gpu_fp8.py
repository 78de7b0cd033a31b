"""GPU parity of the FP8 E4M3 path against the CPU oracle (through the C ABI).

The codes are the E4M3 format of "DeepSeek V4 '950' unified FP8 dataflow"
(sec. 2.1); its FP8 products feed an FP32 accumulator (sec. 2.3).  The oracle
accumulates exactly.  The library offers two ways to multiply the codes:

* CODE_FP8 (the default): every code is decoded to bf16 (exactly: E4M3
  values have at most 4 significant bits) and multiplied on the bf16 matrix
  cores, whose products are exact in fp32 and summed in fp32 -- the pages'
  fp32 accumulator.  A product chain has at most K/16 + 5 fp32 additions (an
  instruction sums 16 or 32 products, at most 5 levels, then adds them to the
  running accumulator), so per output

      |acc - exact| <= (K/16 + 5) * 2^-24 * sum_k |a_k b_k|.

  This path is held to the INT8 path's bar on y.
* CODE_FP8_FAST: gfx950's FP8 matrix cores, which do not accumulate exactly.
  A probe of single v_mfma_scale_f32_16x16x128_f8f6f4 and _32x32x64_f8f6f4
  instructions (a product 256 * 256 = 2^16 next to small ones) shows how one
  instruction sums: its products are taken in groups of 8 consecutive k;
  inside a group every product is cut to a multiple of 2^(e - 13), e the
  exponent of the group's largest product (2^16 + 8 is kept, 2^16 + 4 and
  2^16 + 7 lose their low bits; 40 products of 4 next to 2^16 lose only the 7
  in its group), and the group sums and the accumulator between instructions
  are fp32-accurate.  Its bound, per output:

      sum over groups g of (nonzero products in g - 1) * 2^(floor(log2 max_g) - 13)
        + (K/8 + K/64 + 1) * 2^-24 * sum_k |a_k b_k|

  (the second term: one fp32 rounding for each group sum and instruction
  added).  This path misses the 1e-3 bar on y on the tiled shapes -- an h code
  that moved one E4M3 step shifts a product by up to 1/8 of its size -- and
  those checks are reported as expected failures with the measured figures.

For both, scaled by the operands' scales, plus the epilogue's roundings:

* per-row quantisation codes and scales: bit-exact (same fp32 quotient, round
  to nearest even);
* every E4M3 value through the GEMM: exact (one nonzero product per output);
* GEMM outputs within the path's bound;
* MoE layer: x codes exact, routing as in the INT8 path (same fp32 router), h
  within the bound its accumulators imply, every h code a correct rounding of
  some value inside that bound (so a code differs from the oracle's only next
  to a rounding midpoint), o and y within the bounds that follow; then the
  spec bar of the INT8 path on y (error <= 1e-3 of sum_j |o_j| and of
  the row maximum, on every token routed like the oracle's).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import Y_TOL, near_tie_tokens, sum_rel_metric, to_np, valid_topk

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
GROUP = 8          # products aligned together inside one FP8 MFMA
KEEP_BITS = 13     # bits kept below the group's largest product


def f32_sum_bound(w_abs, x_abs):
    """(bound, sum |products|) of the dot products w_abs[n] . x_abs (decoded
    E4M3 magnitudes, float64) for exact products summed in fp32 along chains
    of at most K/16 + 5 additions (the CODE_FP8 path)."""
    K = w_abs.shape[1]
    S = w_abs @ x_abs
    return (K / 16 + 5) * U * S, S


def mfma_fp8_bound(w_abs, x_abs):
    """(bound, sum |products|) of the dot products w_abs[n] . x_abs (decoded
    E4M3 magnitudes, float64; w_abs [N, K], x_abs [K]) under the instruction
    model above: the truncation inside each group of 8 consecutive k, and one
    fp32 rounding per group sum and per instruction."""
    N, K = w_abs.shape
    p = (w_abs * x_abs[None, :]).reshape(N, K // GROUP, GROUP)
    mx = p.max(axis=2)
    nnz = (p > 0).sum(axis=2)
    e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
    trunc = np.where(mx > 0, np.maximum(nnz - 1, 0) * np.exp2(e - KEEP_BITS), 0.0).sum(axis=1)
    S = p.sum(axis=(1, 2))
    return trunc + (K / 8 + K / 64 + 1) * U * S, S


@pytest.fixture(scope="module")
def w8():
    import w8a8_quantized_moe_amd as w8mod
    return w8mod


def _midpoint_row():
    """A row whose scale is 1 (its maximum is 448) and whose other values sit
    on E4M3 rounding midpoints, one fp32 ulp either side of them, in the
    subnormal range and at zero."""
    vals = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (0.5 * (vals[:-1] + vals[1:])).astype(np.float32)
    lo = np.nextafter(mids, np.float32(0))
    hi = np.nextafter(mids, np.float32(1e9))
    row = np.concatenate([[448.0], mids, -mids, lo, -hi, hi, [0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    row = row.astype(np.float32)
    pad = (-row.size) % 4
    return np.concatenate([row, np.zeros(pad, np.float32)])


@pytest.mark.parametrize("rows,cols", [(1, 4), (3, 100), (33, 1024), (7, 1028), (5, 4096), (4, 8192),
                                       (2, 10001)])
def test_fp8_quantize_rows_bitexact(w8, rows, cols):
    print(f"fp8 quantize rows={rows} cols={cols}", flush=True)
    g = torch.Generator().manual_seed(rows * 7 + cols)
    x = torch.randn(rows, cols, generator=g)
    x[:, :: max(1, cols // 13)] *= 30.0
    q, s = w8.quantize_rows(x.cuda(), code=w8.CODE_FP8)
    qo, so = oracle.quantize_rows_fp8(x.numpy())
    assert np.array_equal(to_np(s), so)
    assert np.array_equal(to_np(q), qo)


def test_fp8_quantize_rounding_midpoints_and_subnormals(w8):
    row = _midpoint_row()
    x = np.stack([row, -row, row * np.float32(2.0 ** -20), np.zeros_like(row)])
    q, s = w8.quantize_rows(torch.from_numpy(x).cuda(), code=1)
    qo, so = oracle.quantize_rows_fp8(x)
    assert np.array_equal(to_np(s), so)
    bad = np.argwhere(to_np(q) != qo)
    assert bad.size == 0, [(int(r), int(c), float(x[r, c]), int(to_np(q)[r, c]), int(qo[r, c]))
                           for r, c in bad[:8]]


def _bound_fn(fast):
    return mfma_fp8_bound if fast else f32_sum_bound


def _fp8_gemm_bound(a_codes, b_codes, s_a, s_b, ref, fast):
    """Per-element bound of the GPU's FP8 GEMM against the exact one."""
    A = np.abs(oracle.e4m3_decode(a_codes)).astype(np.float64)
    B = np.abs(oracle.e4m3_decode(b_codes)).astype(np.float64)
    acc_b = np.stack([_bound_fn(fast)(B, A[m])[0] for m in range(A.shape[0])])
    return acc_b * (s_a[:, None].astype(np.float64) * s_b[None, :]) + 4 * U * np.abs(ref.astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (100, 256, 384), (257, 384, 1024), (300, 256, 2048),
                                   (513, 640, 4096),
                                   # last m-tiles of 128 and 74 rows on 256-wide tiles (the half-tile
                                   # schedule: all eight waves on those rows)
                                   (384, 512, 256), (330, 768, 640)])
@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast"])
def test_fp8_gemm_within_accumulation_bound(w8, M, N, K, fast):
    print(f"fp8 gemm M={M} N={N} K={K} fast={fast}", flush=True)
    g = torch.Generator().manual_seed(M + N + K)
    a = torch.randn(M, K, generator=g)
    b = torch.randn(N, K, generator=g) * 0.05
    aq, sa = oracle.quantize_rows_fp8(a.numpy())
    bq, sb = oracle.quantize_rows_fp8(b.numpy())
    out = w8.gemm(torch.from_numpy(aq).cuda(), torch.from_numpy(sa).cuda(),
                  w8.pack_weights(torch.from_numpy(bq).cuda()), torch.from_numpy(sb).cuda(), N, K,
                  fp8_fast=fast)
    got = to_np(out).astype(np.float64)
    ref = oracle.dense_fp8(aq, sa, bq, sb)
    bound = _fp8_gemm_bound(aq, bq, sa, sb, ref, fast)
    err = np.abs(got - ref)
    print(f"  max err / bound {float((err / bound).max()):.3f}", flush=True)
    assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast"])
def test_fp8_gemm_decodes_every_code(w8, fast):
    """Each of the 254 finite E4M3 codes as the only nonzero product of an
    output (at every byte position of a 128-k row, against 1.0 = 0x38): the
    GEMM must return its value exactly -- the decoding of every code, in
    every operand lane position, pinned to the format's definition."""
    M, N, K = 256, 128, 128
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0  # the two NaN codes
    aq = np.zeros((M, K), np.uint8)
    aq[np.arange(M), np.arange(M) % K] = codes
    bq = np.full((N, K), 0x38, np.uint8)
    ones = np.ones(M, np.float32)
    out = w8.gemm(torch.from_numpy(aq).cuda(), torch.from_numpy(ones).cuda(),
                  w8.pack_weights(torch.from_numpy(bq).cuda()), torch.ones(N, device="cuda"), N, K,
                  fp8_fast=fast)
    got = to_np(out)
    want = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(got, np.repeat(want[:, None], N, axis=1))


def _codes(t):
    return to_np(t).view(np.uint8)


class _Decoded:
    """Decoded E4M3 weight matrices of one expert at a time (a whole layer of
    decoded fp64 weights would not fit in host memory at the larger shapes)."""

    def __init__(self, codes):
        self.codes = codes
        self.cache = {}

    def __getitem__(self, e):
        if e not in self.cache:
            if len(self.cache) > 2:
                self.cache.clear()
            self.cache[e] = np.abs(oracle.e4m3_decode(self.codes[e]))
        return self.cache[e]


_MODES = {"dynamic": 0, "clipped": 1, "static": 2}


def check_moe_fp8(w8, inp, tokens=None, qopts=None, fast=False):
    """qopts: the x quantisation options by their oracle names (x_smooth as a
    numpy vector, x_scale_mode, x_clip); the gate-up weights then take
    1/x_smooth on their input channels on both sides.  fast: the layer on the
    FP8 matrix cores (CODE_FP8_FAST), else exact products summed in fp32."""
    bound = _bound_fn(fast)
    want_code = w8.CODE_FP8_FAST if fast else w8.CODE_FP8
    T, H, E, k, I = inp["T"], inp["H"], inp["E"], inp["k"], inp["I"]
    qopts = qopts or {}
    sm = qopts.get("x_smooth")
    if "w_gu_f32" in inp:
        kw = {}
        if qopts:
            kw = dict(x_smooth=None if sm is None else torch.from_numpy(sm).cuda(),
                      x_scale_mode=_MODES[qopts.get("x_scale_mode", "dynamic")],
                      x_clip=qopts.get("x_clip", 0.0))
        wts, codes = w8.MoEWeights.from_fp32(inp["wr"], inp["b"], inp["w_gu_f32"], inp["w_d_f32"],
                                             keep_codes=True, code=want_code, **kw)
        twoI = 2 * I
        if sm is None:
            qg, sg = oracle.quantize_rows_fp8(to_np(inp["w_gu_f32"]).reshape(E * twoI, H))
        else:
            qg, sg = oracle.quantize_rows_ex(to_np(inp["w_gu_f32"]).reshape(E * twoI, H),
                                             col_mul=np.float32(1.0) / sm, code="fp8")
        qd, sd = oracle.quantize_rows_fp8(to_np(inp["w_d_f32"]).reshape(E * H, I))
        # offline weight quantisation: exact
        assert np.array_equal(_codes(codes["w_gu"]).reshape(-1, H), qg)
        assert np.array_equal(_codes(codes["w_d"]).reshape(-1, I), qd)
        assert np.array_equal(to_np(codes["s_gu"]).reshape(-1), sg)
        assert np.array_equal(to_np(codes["s_d"]).reshape(-1), sd)
        oc = dict(w_gu=qg.reshape(E, twoI, H), s_gu=sg.reshape(E, twoI), w_d=qd.reshape(E, H, I),
                  s_d=sd.reshape(E, H))
    else:
        assert not qopts
        wts = w8.MoEWeights.from_int8(inp["wr"], inp["b"], inp["w_gu"], inp["s_gu"], inp["w_d"],
                                      inp["s_d"], fp8_fast=fast)
        oc = {n: to_np(inp[n]) for n in ("w_gu", "s_gu", "w_d", "s_d")}
    assert wts.code == want_code
    print(f"fp8 moe T={T} H={H} E={E} k={k} I={I} fast={fast}", flush=True)
    lay = w8.moe_workspace_layout(T, H, E, k, I)
    ws = torch.empty((lay["total_bytes"],), dtype=torch.uint8, device="cuda")
    y = w8.moe_forward(inp["x"], wts, k, workspace=ws)
    torch.cuda.synchronize()
    g = {n: to_np(v) for n, v in w8.workspace_views(ws, T, H, E, k, I).items()}
    y = to_np(y)
    x = to_np(inp["x"])
    o = oracle.moe_forward(x, to_np(inp["wr"]), to_np(inp["b"]), oc["w_gu"], oc["s_gu"], oc["w_d"],
                           oc["s_d"], k, tokens=tokens, want_h=True, want_acc=True, code="fp8", **qopts)
    tok = o["tokens"]
    # 1. activation codes and scales: exact
    assert np.array_equal(g["x_q"].view(np.uint8), o["x_q"])
    assert np.array_equal(g["x_scale"], o["s_x"])
    # 2-4. routing: the fp32 router of the INT8 path, checked the same way
    assert valid_topk(g["logits"], g["topk_ids"]).all()
    flag = near_tie_tokens(o["logits"], g["logits"], k)
    same = np.all(g["topk_ids"] == o["ids"], axis=1)
    assert np.all(same | flag)
    dl = np.abs(g["logits"].astype(np.float64) - o["logits"]).max(axis=1)
    inv = np.empty(T * k, np.int64)
    inv[g["sorted_assign"]] = np.arange(T * k)
    a_rows = (tok[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    ok = np.repeat(same[tok], k)
    rows_g = inv[a_rows]
    a_tok = np.repeat(tok, k)
    ids = o["ids"][tok].reshape(-1)
    # 5. h: exact maths on the oracle side, fp32 accumulators on the GPU; the
    #    bound follows the accumulators' error through the scaling and SwiGLU
    xa = np.abs(oracle.e4m3_decode(o["x_q"][a_tok])).astype(np.float64)
    wgu = _Decoded(oc["w_gu"])
    # the accumulators' bound (code units), per output
    AB = np.stack([bound(wgu[e], xa[r])[0] for r, e in enumerate(ids)])
    sc = o["s_x"][a_tok].astype(np.float64)[:, None] * oc["s_gu"][ids]
    gv = o["acc_gu"][:, :I] * sc[:, :I]
    uv = o["acc_gu"][:, I:] * sc[:, I:]
    dg = AB[:, :I] * sc[:, :I] + 6 * U * np.abs(gv)
    du = AB[:, I:] * sc[:, I:] + 6 * U * np.abs(uv)
    sig = 1.0 / (1.0 + np.exp(-np.clip(gv, -700, 700)))
    dsilu = np.abs(sig * (1 + gv * (1 - sig))) + 1e-3
    h_o = o["h"].astype(np.float64)
    hb = dsilu * np.abs(uv) * dg + np.abs(gv * sig) * du + dg * du + 8 * U * np.abs(h_o) + 1e-37
    h_g = g["h"][rows_g].astype(np.float64)
    assert np.all((np.abs(h_g - h_o) <= hb)[ok]), float((np.abs(h_g - h_o) / hb)[ok].max())
    # 6. h codes: the scale follows the row maximum; every GPU code is the
    #    rounding of a value inside the bound (codes are monotone in the value,
    #    so it lies between the codes of the bound's two ends)
    sh_g = g["h_scale"][rows_g].astype(np.float64)
    sh_o = o["s_h"].astype(np.float64)
    amax_b = np.max(hb, axis=1)
    assert np.all((np.abs(sh_g - sh_o) <= amax_b / 448.0 + 2 * U * sh_o)[ok])
    hq_g = g["h_q"].view(np.uint8)[rows_g]
    hq_o = o["h_q"]
    slack = 1.0 + 4 * U
    lo = np.where(sh_g[:, None] > 0, (h_o - hb * slack) / sh_g[:, None], 0.0)
    hi = np.where(sh_g[:, None] > 0, (h_o + hb * slack) / sh_g[:, None], 0.0)
    v_lo = oracle.e4m3_decode(oracle.e4m3_encode(np.clip(lo, -448, 448).astype(np.float32)))
    v_hi = oracle.e4m3_decode(oracle.e4m3_encode(np.clip(hi, -448, 448).astype(np.float32)))
    v_g = oracle.e4m3_decode(hq_g)
    inside = (v_lo <= v_g) & (v_g <= v_hi)
    assert np.all(inside[ok]), int((~inside[ok]).sum())
    differ = (v_g != oracle.e4m3_decode(hq_o)) & ok[:, None]
    # (the scales may differ in their last bits: the row maximum carries the
    # accumulation error; that moves o by a relative 2^-23 at most)
    rows_exact = ~differ.any(axis=1) & ok
    print(f"  h codes differing: {int(differ.sum())} of {int(ok.sum()) * I}; "
          f"rows with all codes equal: {int(rows_exact.sum())} of {int(ok.sum())}; "
          f"rows with equal scales: {int(((sh_g == sh_o) & ok).sum())}", flush=True)
    # 7. o = w * v: bound from the weights' error, the h codes that moved and
    #    the down GEMM's fp32 accumulation
    hv_g = v_g * sh_g[:, None]
    hv_o = oracle.e4m3_decode(hq_o) * sh_o[:, None]
    dh = np.abs(hv_g - hv_o)
    wd = _Decoded(oc["w_d"])
    hga = np.abs(v_g)
    sd = oc["s_d"][ids]
    v_o = o["acc_d"] * sh_o[:, None] * sd
    dv = np.stack([wd[e] @ dh[r] for r, e in enumerate(ids)]) * sd \
        + np.stack([bound(wd[e], hga[r].astype(np.float64))[0] for r, e in enumerate(ids)]) \
        * sh_g[:, None] * sd + 6 * U * np.abs(v_o)
    w_g = g["topk_w"][tok].reshape(-1).astype(np.float64)
    w_o = o["w"][tok].reshape(-1).astype(np.float64)
    assert np.all((np.abs(w_g - w_o) <= np.abs(w_o) * (4 * np.repeat(dl[tok], k) + 2e-6))[ok])
    ob = np.abs(w_g)[:, None] * dv + np.abs(w_g - w_o)[:, None] * np.abs(v_o) \
        + 2 * U * np.abs(o["o"])
    o_g = g["o"][a_rows].astype(np.float64)
    assert np.all((np.abs(o_g - o["o"]) <= ob)[ok]), float((np.abs(o_g - o["o"]) / ob)[ok].max())
    # 8. y: within the sum of the o bounds
    yt = same[tok]
    terms = np.abs(o["o"]).reshape(len(tok), k, H).sum(axis=1)
    yb = ob.reshape(len(tok), k, H).sum(axis=1) + 2 * k * U * terms
    assert np.all((np.abs(y[tok].astype(np.float64) - o["y"]) <= yb)[yt])
    # The spec bar, exactly as the INT8 path applies it: on every token
    # routed like the oracle's, error <= 1e-3 of sum_j |o_j| per element and of
    # the row maximum.
    sr, mx = sum_rel_metric(y[tok][yt], o["y"][yt], terms[yt]) if yt.any() else (0.0, 0.0)
    te = yt & rows_exact.reshape(len(tok), k).all(axis=1)
    sr_eq, mx_eq = sum_rel_metric(y[tok][te], o["y"][te], terms[te]) if te.any() else (0.0, 0.0)
    print(f"  y: sum-relative {sr:.2e}, row-max {mx:.2e} on {int(yt.sum())} tokens; on the "
          f"{int(te.sum())} whose h codes all equal the oracle's: {sr_eq:.2e}, {mx_eq:.2e}", flush=True)
    if not fast:
        assert sr <= Y_TOL and mx <= Y_TOL, (sr, mx)
    elif sr > Y_TOL or mx > Y_TOL:
        pytest.xfail(f"FP8 layer misses the 1e-3 bar on y: sum-relative {sr:.2e}, row-max {mx:.2e} "
                     f"({int(differ.sum())} h codes moved one E4M3 step next to a rounding midpoint; "
                     f"the derived bounds above hold)")
    return g, o


@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast"])
def test_fp8_moe_tiny_fp32_weights(w8, fast):
    """The tiny layer with its fp32 expert weights quantised to E4M3 by each
    side (the skinny GEMM path: few rows per expert)."""
    check_moe_fp8(w8, synth.moe_inputs("tiny", device="cuda"), fast=fast)


@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast"])
def test_fp8_moe_tiled_path(w8, fast):
    """Enough rows per expert for the LDS-tiled grouped GEMM (A > 4E),
    ragged segments, fp32 weights quantised by each side."""
    inp = synth.moe_inputs("edge", device="cuda", T=300, H=256, E=8, k=2, I=256, n_outlier=2,
                           outlier_scale=20.0, bf16_x=False, bias="zero", weights="fp32")
    check_moe_fp8(w8, inp, fast=fast)


@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast"])
def test_fp8_moe_decode_shape_sampled(w8, fast):
    """The decode layer's shape with E4M3 weight codes drawn directly."""
    inp = synth.moe_inputs("decode", device="cuda", weights="fp8")
    check_moe_fp8(w8, inp, tokens=np.array([0, 1, 17, 33, 62, 63]), fast=fast)


@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast"])
def test_fp8_moe_prefill_shape_sampled(w8, fast):
    """The prefill layer's shape (skewed routing, tiled GEMMs) with E4M3 codes."""
    inp = synth.moe_inputs("prefill", device="cuda", weights="fp8")
    check_moe_fp8(w8, inp, tokens=np.array([0, 5, 1000, 4096, 8191]), fast=fast)


@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast"])
def test_fp8_moe_large_shape_sampled(w8, fast):
    """The large layer's shape (E=256, top-8, H=7168, I=2048) with E4M3 codes,
    checked on a few tokens (each touches 8 experts)."""
    inp = synth.moe_inputs("large", device="cuda", weights="fp8")
    check_moe_fp8(w8, inp, tokens=np.array([0, 7777, 16383]), fast=fast)


@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast"])
def test_fp8_moe_ragged_narrow_hidden(w8, fast):
    """E4M3 codes with H = 384 (the down GEMM on 256x128 tiles), ragged T and a
    segment mix of full, partial and half m-tiles."""
    inp = synth.moe_inputs("edge", device="cuda", T=713, H=384, E=5, k=3, I=384, n_outlier=2,
                           outlier_scale=20.0, bf16_x=False, bias="zero", weights="fp32")
    check_moe_fp8(w8, inp, fast=fast)


@pytest.mark.parametrize("mode", ["clipped", "static"])
def test_fp8_moe_with_scale_options(w8, mode):
    """E4M3 codes with a smoothing vector on x (the gate-up weights quantised
    with its inverse) and a clipped or static x scale: x codes and scales
    exact, the rest within the FP8 bounds above."""
    inp = synth.moe_inputs("edge", device="cuda", T=300, H=256, E=8, k=2, I=256, n_outlier=2,
                           outlier_scale=20.0, bf16_x=False, bias="zero", weights="fp32")
    x = to_np(inp["x"])
    H = inp["H"]
    m = (1.0 / np.sqrt(np.abs(x).max(axis=0) + 1e-3)).astype(np.float32)
    m *= np.random.default_rng(H).uniform(0.9, 1.1, H).astype(np.float32)
    amax = np.abs(x * m).max(axis=1)
    check_moe_fp8(w8, inp, qopts=dict(x_smooth=m, x_scale_mode=mode,
                                      x_clip=float(np.quantile(amax, 0.5))))
