"""CPU oracle for the W8A8 MoE expert layer -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plainly written definition the GPU path is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import it.  It shares no code with the HIP library and
never imports it.

The arithmetic lives in ``oracle.c`` (plain C loops, OpenMP over independent
rows).  This module only marshals numpy arrays to it and strings the steps
together in the order the pages give them:

  per-token quant -> fp32 router -> softmax/top-k/renormalise -> permute into
  per-expert segments -> gate-up GEMM + dequant + SiLU*up + requant -> down
  GEMM + dequant * routing weight -> combine.

With FP8 codes (DeepSeek V4 page, sec. 2.1 and 2.3) the codes are E4M3 and
the accumulators exact (fp64), rounded once to fp32 before the epilogue.

Sources: "W8A8 quantisation of MiniMax-M3 on K100AI" sec. 2.1 (quant maths,
scale outer product in the GEMM epilogue); "Tencent Hunyuan AI Infra ...
Hopper" sec. 1.3 (FusedMoE stage list, weighted aggregation at the end);
"DeepSeek V4 '950' unified FP8 dataflow" sec. 2.3 (wide accumulator, output
requantised), sec. 2.4 (per-output-channel weight scales), sec. 4.1 (router in
full precision).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA
    contraction, so every fp32 operation is one IEEE-rounded step)."""
    cmd = [
        "gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
        "-fvisibility=hidden", _SRC, "-o", _SO + ".tmp", "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_quantize_rows.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_gemm_i32.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_dense_w8a8.argtypes = [P, P, P, P, I64, I64, I64, P]
    lib.oracle_router_logits.argtypes = [P, P, P, I64, I64, I64, P]
    lib.oracle_topk_softmax.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_permute.argtypes = [P, I64, I64, I64, P, P, P]
    lib.oracle_silu.argtypes = [ctypes.c_float]
    lib.oracle_silu.restype = ctypes.c_float
    lib.oracle_expert_ffn.argtypes = [I64, P, P, P, P, P, I64, I64, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_combine.argtypes = [P, I64, I64, I64, P]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_quantize_rows_fp8.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_gemm_fp8.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_dense_fp8.argtypes = [P, P, P, P, I64, I64, I64, P]
    lib.oracle_expert_ffn_fp8.argtypes = [I64, P, P, P, P, P, I64, I64, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_quantize_rows_ex.argtypes = [P, I64, I64, I64, P, ctypes.c_int, ctypes.c_float,
                                            ctypes.c_int, P, P]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


# --------------------------------------------------------------------------
# single steps
# --------------------------------------------------------------------------
def quantize_rows(x):
    """Per-row symmetric INT8 quantisation (K100AI page, sec. 2.1).
    x: [rows, cols] float32 -> (q int8 [rows, cols], s float32 [rows])."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows,), np.float32)
    _load().oracle_quantize_rows(_p(x), rows, cols, cols, _p(q), _p(s))
    return q, s


def gemm_i32(a, b):
    """acc = a @ b.T exactly in int32; a [M, K] int8, b [N, K] int8."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    _load().oracle_gemm_i32(_p(a), _p(b), M, N, K, _p(acc))
    return acc


def dense_w8a8(a_q, s_a, b_q, s_b):
    """Dense W8A8 GEMM with the per-token x per-channel scale outer product
    applied to the int32 result (K100AI page, sec. 2.1)."""
    a_q = _c(a_q, np.int8)
    b_q = _c(b_q, np.int8)
    s_a = _c(s_a, np.float32)
    s_b = _c(s_b, np.float32)
    M, K = a_q.shape
    N = b_q.shape[0]
    out = np.empty((M, N), np.float32)
    _load().oracle_dense_w8a8(_p(a_q), _p(s_a), _p(b_q), _p(s_b), M, N, K, _p(out))
    return out


def router_logits(x, wr, bias=None):
    """fp64 router logits on the unquantised activations (DeepSeek V4 page,
    sec. 4.1).  x [T, H] f32, wr [E, H] f32, bias [E] f32 or None."""
    x = _c(x, np.float32)
    wr = _c(wr, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float64)
    _load().oracle_router_logits(_p(x), _p(wr), _p(b), T, H, E, _p(out))
    return out


def topk_softmax(logits, k):
    """softmax -> top-k (descending, ties to the lower index) -> renormalise."""
    logits = _c(logits, np.float64)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().oracle_topk_softmax(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def permute(ids, E):
    """Contiguous per-expert segments, ascending token order inside each.
    Returns (counts [E], offsets [E+1], sorted_assign [T*k]) with entries
    a = t*k + j."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty((E,), np.int32)
    offsets = np.empty((E + 1,), np.int32)
    sorted_assign = np.empty((T * k,), np.int32)
    _load().oracle_permute(_p(ids), T, k, E, _p(counts), _p(offsets), _p(sorted_assign))
    return counts, offsets, sorted_assign


def silu(g):
    """SiLU in fp32 with a correctly rounded exponential (elementwise)."""
    lib = _load()
    g = np.asarray(g, np.float32)
    out = np.empty_like(g)
    flat_in = g.reshape(-1)
    flat_out = out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_silu(float(flat_in[i]))
    return out


def expert_ffn(a_token, a_expert, a_weight, x_q, s_x, w_gu, s_gu, w_d, s_d, want_acc=False,
               want_h=False):
    """Expert SwiGLU FFN for a list of assignments (see oracle.c)."""
    a_token = _c(a_token, np.int64)
    a_expert = _c(a_expert, np.int32)
    a_weight = _c(a_weight, np.float32)
    x_q = _c(x_q, np.int8)
    s_x = _c(s_x, np.float32)
    w_gu = _c(w_gu, np.int8)
    s_gu = _c(s_gu, np.float32)
    w_d = _c(w_d, np.int8)
    s_d = _c(s_d, np.float32)
    n = a_token.shape[0]
    E, twoI, H = w_gu.shape
    I = twoI // 2
    assert w_d.shape == (E, H, I)
    acc_gu = np.empty((n, 2 * I), np.int32) if want_acc else None
    acc_d = np.empty((n, H), np.int32) if want_acc else None
    h = np.empty((n, I), np.float32) if want_h else None
    h_q = np.empty((n, I), np.int8)
    s_h = np.empty((n,), np.float32)
    o = np.empty((n, H), np.float32)
    _load().oracle_expert_ffn(n, _p(a_token), _p(a_expert), _p(a_weight), _p(x_q), _p(s_x), H, I,
                              _p(w_gu), _p(s_gu), _p(w_d), _p(s_d), _p(acc_gu), _p(h), _p(h_q),
                              _p(s_h), _p(acc_d), _p(o))
    out = dict(h_q=h_q, s_h=s_h, o=o)
    if want_acc:
        out["acc_gu"] = acc_gu
        out["acc_d"] = acc_d
    if want_h:
        out["h"] = h
    return out


def combine(o, T, k):
    """y[t] = sum_j o[t*k + j] in j order (fp32)."""
    o = _c(o, np.float32)
    H = o.shape[1]
    y = np.empty((T, H), np.float32)
    _load().oracle_combine(_p(o), T, k, H, _p(y))
    return y


# --------------------------------------------------------------------------
# FP8 E4M3 codes (DeepSeek V4 page, sec. 2.1 and 2.3)
# --------------------------------------------------------------------------
def e4m3_decode(codes):
    """Values of E4M3 codes (uint8 array) as float64."""
    lib = _load()
    c = np.asarray(codes, np.uint8)
    table = np.array([lib.oracle_e4m3_decode(i) for i in range(256)], np.float64)
    return table[c]


def e4m3_encode(v):
    """Nearest E4M3 codes of float32 values (ties to even, saturating)."""
    lib = _load()
    v = np.asarray(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    fi, fo = v.reshape(-1), out.reshape(-1)
    for i in range(fi.size):
        fo[i] = lib.oracle_e4m3_encode(float(fi[i]))
    return out


def quantize_rows_fp8(x):
    """Per-row FP8 E4M3 quantisation: s = max|x|/448, code = E4M3(x/s).
    x: [rows, cols] float32 -> (q uint8 [rows, cols], s float32 [rows])."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows,), np.float32)
    _load().oracle_quantize_rows_fp8(_p(x), rows, cols, cols, _p(q), _p(s))
    return q, s


SCALE_MODES = {"dynamic": 0, "clipped": 1, "static": 2}


def quantize_rows_ex(x, col_mul=None, mode="dynamic", clip=0.0, code="int8"):
    """Per-row quantisation with an optional per-column factor (SmoothQuant,
    K100AI page sec. 2.2) and a clipped or static scale (K100AI sec. 2.2,
    DeepSeek V4 page sec. 3.1); see oracle.c.  Returns (codes, scales)."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, cols = x.shape
    m = None if col_mul is None else _c(col_mul, np.float32)
    assert m is None or m.shape == (cols,)
    fp8 = code == "fp8"
    q = np.empty((rows, cols), np.uint8 if fp8 else np.int8)
    s = np.empty((rows,), np.float32)
    _load().oracle_quantize_rows_ex(_p(x), rows, cols, cols, None if m is None else _p(m),
                                    SCALE_MODES[mode], float(clip), int(fp8), _p(q), _p(s))
    return q, s


def gemm_fp8(a, b):
    """Exact accumulator sum_k E4M3(a) * E4M3(b) in float64; a [M, K], b [N, K] uint8 codes."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    acc = np.empty((M, N), np.float64)
    _load().oracle_gemm_fp8(_p(a), _p(b), M, N, K, _p(acc))
    return acc


def dense_fp8(a_q, s_a, b_q, s_b):
    """Dense GEMM with FP8 codes: ((float)acc * s_a) * s_b."""
    a_q = _c(a_q, np.uint8)
    b_q = _c(b_q, np.uint8)
    s_a = _c(s_a, np.float32)
    s_b = _c(s_b, np.float32)
    M, K = a_q.shape
    N = b_q.shape[0]
    out = np.empty((M, N), np.float32)
    _load().oracle_dense_fp8(_p(a_q), _p(s_a), _p(b_q), _p(s_b), M, N, K, _p(out))
    return out


def expert_ffn_fp8(a_token, a_expert, a_weight, x_q, s_x, w_gu, s_gu, w_d, s_d, want_acc=False,
                   want_h=False):
    """Expert SwiGLU FFN with FP8 codes (see oracle.c)."""
    a_token = _c(a_token, np.int64)
    a_expert = _c(a_expert, np.int32)
    a_weight = _c(a_weight, np.float32)
    x_q = _c(x_q, np.uint8)
    s_x = _c(s_x, np.float32)
    w_gu = _c(w_gu, np.uint8)
    s_gu = _c(s_gu, np.float32)
    w_d = _c(w_d, np.uint8)
    s_d = _c(s_d, np.float32)
    n = a_token.shape[0]
    E, twoI, H = w_gu.shape
    I = twoI // 2
    assert w_d.shape == (E, H, I)
    acc_gu = np.empty((n, 2 * I), np.float64) if want_acc else None
    acc_d = np.empty((n, H), np.float64) if want_acc else None
    h = np.empty((n, I), np.float32) if want_h else None
    h_q = np.empty((n, I), np.uint8)
    s_h = np.empty((n,), np.float32)
    o = np.empty((n, H), np.float32)
    _load().oracle_expert_ffn_fp8(n, _p(a_token), _p(a_expert), _p(a_weight), _p(x_q), _p(s_x), H, I,
                                  _p(w_gu), _p(s_gu), _p(w_d), _p(s_d), _p(acc_gu), _p(h), _p(h_q),
                                  _p(s_h), _p(acc_d), _p(o))
    out = dict(h_q=h_q, s_h=s_h, o=o)
    if want_acc:
        out["acc_gu"] = acc_gu
        out["acc_d"] = acc_d
    if want_h:
        out["h"] = h
    return out


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------
def moe_forward(x, wr, bias, w_gu_q, s_gu, w_d_q, s_d, k, tokens=None, want_acc=False,
                want_h=False, route_tokens=None, code="int8", x_smooth=None, x_scale_mode="dynamic",
                x_clip=0.0):
    """The W8A8 MoE expert layer, step by step.

    x      [T, H]   float32 activations
    wr     [E, H]   float32 router weight, bias [E] float32 or None
    w_gu_q [E, 2I, H] int8 (rows 0..I-1 gate, I..2I-1 up), s_gu [E, 2I] f32
    w_d_q  [E, H, I]  int8, s_d [E, H] f32
    code   "int8" (the codes above are int8) or "fp8" (uint8 E4M3 codes; the
           activations and h are then quantised to E4M3 as well)
    x_smooth, x_scale_mode, x_clip: the activation quantisation options of
           quantize_rows_ex (the weights' input channels then carry the
           inverse factor; the router reads the unsmoothed x)

    ``tokens``: optional sorted subset of token indices for which the expert
    FFN, the outputs o and y are computed (tokens are independent, so a
    subset's rows equal the same rows of a full run).  Routing and the
    permutation always cover all tokens, unless ``route_tokens`` restricts
    the whole layer to those rows (then T is their number).
    Returns a dict of every intermediate, keyed by (t, j) order for per-
    assignment tensors.
    """
    x = _c(x, np.float32)
    if route_tokens is not None:
        x = x[np.asarray(route_tokens)]
    T, H = x.shape
    E = wr.shape[0]
    assert code in ("int8", "fp8")
    if x_smooth is None and x_scale_mode == "dynamic":
        x_q, s_x = quantize_rows(x) if code == "int8" else quantize_rows_fp8(x)
    else:
        x_q, s_x = quantize_rows_ex(x, x_smooth, x_scale_mode, x_clip, code)
    logits = router_logits(x, wr, bias)
    ids, w = topk_softmax(logits, k)
    counts, offsets, sorted_assign = permute(ids, E)
    if tokens is None:
        tok = np.arange(T, dtype=np.int64)
    else:
        tok = np.asarray(tokens, np.int64)
    a_token = np.repeat(tok, k)
    a_expert = ids[tok].reshape(-1)
    a_weight = w[tok].reshape(-1)
    ffn = (expert_ffn if code == "int8" else expert_ffn_fp8)(
        a_token, a_expert, a_weight, x_q, s_x, w_gu_q, s_gu, w_d_q, s_d, want_acc=want_acc,
        want_h=want_h)
    y = combine(ffn["o"], tok.shape[0], k)
    res = dict(x_q=x_q, s_x=s_x, logits=logits, ids=ids, w=w, counts=counts, offsets=offsets,
               sorted_assign=sorted_assign, tokens=tok, y=y)
    res.update(ffn)
    return res
