"""Host-side checks of the C ABI (no GPU needed): the shared library loads,
exports every function include/w8a8moe.h declares with the argument count the
Python binding marshals, and rejects bad arguments on the host before any
kernel is enqueued."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8moe.h")
LIB = os.path.join(ROOT, "w8a8_quantized_moe_amd", "libw8a8moe.so")


def _ensure_built():
    if not os.path.exists(LIB):
        subprocess.run([sys.executable, os.path.join(ROOT, "w8a8_quantized_moe_amd", "build.py")],
                       check=True)


_ensure_built()
from w8a8_quantized_moe_amd import _lib  # noqa: E402  (needs the library)

lib = _lib.lib


def header_functions():
    """{name: number of parameters} of every W8A8_API function in the header."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"W8A8_API\s+[\w\s\*]+?\b(w8a8_\w+)\s*\(([^)]*)\)\s*;", text):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else len(params.split(","))
    return out


def exported_symbols():
    res = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True)
    return {line.split()[-1] for line in res.stdout.splitlines() if " T " in line}


def test_header_parses():
    fns = header_functions()
    assert len(fns) == 18, sorted(fns)


def test_every_declared_function_is_exported():
    syms = exported_symbols()
    missing = [f for f in header_functions() if f not in syms]
    assert not missing, missing


def test_only_declared_functions_are_exported():
    extra = sorted(s for s in exported_symbols() if s.startswith("w8a8") and s not in header_functions())
    assert not extra, extra


def test_binding_matches_header():
    fns = header_functions()
    assert set(_lib.SIGNATURES) == set(fns)
    for name, nparams in fns.items():
        assert len(_lib.SIGNATURES[name][1]) == nparams, name


def test_status_strings_and_version():
    names = {0: "W8A8_OK", 1: "W8A8_ERR_INVALID_ARGUMENT", 2: "W8A8_ERR_UNSUPPORTED_SHAPE",
             3: "W8A8_ERR_WORKSPACE_TOO_SMALL", 4: "W8A8_ERR_MISALIGNED", 5: "W8A8_ERR_HIP"}
    for code, name in names.items():
        assert lib.w8a8_status_string(code).decode() == name
    assert lib.w8a8_status_string(99).decode() == "W8A8_UNKNOWN_STATUS"
    assert lib.w8a8_abi_version() == 4


def _shape(T, H, E, k, I):
    return _lib.MoeShape(T, H, E, k, I)


def _query(T, H, E, k, I):
    lay = _lib.MoeLayout()
    st = lib.w8a8_moe_workspace_query(ctypes.byref(_shape(T, H, E, k, I)), ctypes.byref(lay))
    return st, lay


@pytest.mark.parametrize("T,H,E,k,I", [(16, 128, 8, 2, 256), (64, 4096, 64, 2, 1536),
                                       (16384, 7168, 256, 8, 2048), (0, 128, 1, 1, 128)])
def test_workspace_layout(T, H, E, k, I):
    st, lay = _query(T, H, E, k, I)
    assert st == 0
    A = T * k
    sizes = dict(x_q=T * H, x_scale=4 * T, logits=4 * T * E, topk_ids=4 * A, topk_w=4 * A,
                 expert_counts=4 * E, expert_offsets=4 * (E + 1), sorted_assign=4 * A,
                 h=4 * A * I, h_q=A * I, h_scale=4 * A, o=4 * A * H)
    spans = sorted((getattr(lay, f), getattr(lay, f) + n, f) for f, n in sizes.items())
    for (a0, a1, fa), (b0, _, fb) in zip(spans, spans[1:]):
        assert a1 <= b0, (fa, fb)          # no overlap
    for f in sizes:
        assert getattr(lay, f) % 256 == 0, f
    assert spans[-1][1] <= lay.internal <= lay.total_bytes


@pytest.mark.parametrize("E,etile", [(256, 128), (200, 128), (100, 128), (64, 64), (50, 64), (24, 32)])
def test_workspace_holds_router_planes_from_2048_tokens(E, etile):
    # from 2048 tokens the router weights are split into three bf16 planes of
    # the expert count padded to whole expert tiles: H * E' * 6 bytes more
    # internal scratch than the per-token growth alone accounts for
    H, k, I = 512, 2, 128
    _, a = _query(2047, H, E, k, I)
    _, b = _query(2048, H, E, k, I)
    _, c = _query(2049, H, E, k, I)
    planes = H * (-(-E // etile) * etile) * 6
    per_token = (c.total_bytes - c.internal) - (b.total_bytes - b.internal)
    assert (b.total_bytes - b.internal) - (a.total_bytes - a.internal) >= planes
    assert per_token < planes


@pytest.mark.parametrize("T,H,E,k,I,status", [
    (16, 100, 8, 2, 256, 2),      # H not a multiple of 128
    (16, 128, 8, 2, 200, 2),      # I not a multiple of 128
    (16, 32768, 8, 2, 256, 2),    # H too large
    (16, 128, 257, 2, 256, 2),    # E > 256
    (16, 128, 8, 9, 256, 2),      # k > 8
    (16, 128, 4, 5, 256, 2),      # k > E
    (16, 128, 8, 0, 256, 2),      # k = 0
    (1 << 22, 128, 8, 8, 256, 2),  # T*k > 2^24
    (1 << 61, 128, 8, 8, 256, 2),  # T*k would overflow int64
    ((1 << 24) + 1, 128, 8, 1, 256, 2),  # T > 2^24
    (-1, 128, 8, 2, 256, 1),      # negative size
])
def test_workspace_query_rejects(T, H, E, k, I, status):
    st, _ = _query(T, H, E, k, I)
    assert st == status
    assert lib.w8a8_last_error().decode()


def test_null_arguments_rejected_before_launch():
    lay = _lib.MoeLayout()
    assert lib.w8a8_moe_workspace_query(None, ctypes.byref(lay)) == 1
    assert lib.w8a8_moe_workspace_query(ctypes.byref(_shape(16, 128, 8, 2, 256)), None) == 1
    # forward with NULL tensors: host check, nothing enqueued
    w = _lib.MoeWeights()
    st = lib.w8a8_moe_forward(ctypes.byref(_shape(16, 128, 8, 2, 256)), ctypes.byref(w), None, None,
                              None, 0, None)
    assert st == 1 and "NULL" in lib.w8a8_last_error().decode()
    # T = 0 is a no-op that touches nothing
    assert lib.w8a8_moe_forward(ctypes.byref(_shape(0, 128, 8, 2, 256)), None, None, None, None, 0,
                                None) == 0


def test_forward_checks_workspace_and_alignment():
    # fake, never dereferenced device addresses: the host checks fail first
    base = 1 << 40
    w = _lib.MoeWeights(base, None, base, base, base, base)
    sh = ctypes.byref(_shape(16, 128, 8, 2, 256))
    st = lib.w8a8_moe_forward(sh, ctypes.byref(w), base, base + 65536, base + 2 * 65536, 16, None)
    assert st == 3 and "workspace" in lib.w8a8_last_error().decode()
    st = lib.w8a8_moe_forward(sh, ctypes.byref(w), base + 4, base + 65536, base + 2 * 65536, 1 << 30,
                              None)
    assert st == 4
    st = lib.w8a8_moe_forward(sh, ctypes.byref(w), base, base + 65536, base + 2 * 65536 + 16, 1 << 30,
                              None)
    assert st == 4
    st = lib.w8a8_moe_forward(sh, ctypes.byref(w), base, base, base + 2 * 65536, 1 << 30, None)
    assert st == 1  # y aliases x
    # partial overlaps: y inside x (16 x 128 fp32 = 8 KiB), y or x inside the workspace
    st = lib.w8a8_moe_forward(sh, ctypes.byref(w), base, base + 4096, base + 2 * 65536, 1 << 30, None)
    assert st == 1 and "overlap x" in lib.w8a8_last_error().decode()
    st = lib.w8a8_moe_forward(sh, ctypes.byref(w), base, base + 2 * 65536 + 1024, base + 2 * 65536,
                              1 << 30, None)
    assert st == 1 and "workspace" in lib.w8a8_last_error().decode()
    st = lib.w8a8_moe_forward(sh, ctypes.byref(w), base + 2 * 65536 + 4096, base, base + 2 * 65536,
                              1 << 30, None)
    assert st == 1 and "workspace" in lib.w8a8_last_error().decode()
    smooth_bad = _lib.MoeWeights(base, None, base, base, base, base, 0, base + 4, 0, 0.0)
    st = lib.w8a8_moe_forward(sh, ctypes.byref(smooth_bad), base, base + 65536, base + 2 * 65536,
                              1 << 30, None)
    assert st == 4  # x_smooth must be 16-byte aligned
    clip_bad = _lib.MoeWeights(base, None, base, base, base, base, 0, None, 2, -1.0)
    st = lib.w8a8_moe_forward(sh, ctypes.byref(clip_bad), base, base + 65536, base + 2 * 65536,
                              1 << 30, None)
    assert st == 1 and "clip" in lib.w8a8_last_error().decode()
    for c in (3, 7, -1):
        bad = _lib.MoeWeights(base, None, base, base, base, base, c)
        st = lib.w8a8_moe_forward(sh, ctypes.byref(bad), base, base + 65536, base + 2 * 65536, 1 << 30,
                                  None)
        assert st == 1 and "code" in lib.w8a8_last_error().decode()  # unknown weight code
    # both FP8 codes pass the code check (the call then stops at the next one)
    for c in (_lib.CODE_FP8, _lib.CODE_FP8_FAST):
        ok = _lib.MoeWeights(base, None, base, base, base, base, c)
        st = lib.w8a8_moe_forward(sh, ctypes.byref(ok), base, base, base + 2 * 65536, 1 << 30, None)
        assert st == 1 and "overlap x" in lib.w8a8_last_error().decode()
    # the gate-up accumulator capture: INT8 codes only, a non-NULL output, a
    # large enough aligned workspace
    acc = lib.w8a8_moe_gate_up_acc
    fp8 = _lib.MoeWeights(base, None, base, base, base, base, 1)
    assert acc(sh, ctypes.byref(w), base + 2 * 65536, 1 << 30, None, None) == 1
    assert acc(sh, ctypes.byref(fp8), base + 2 * 65536, 1 << 30, base, None) == 1
    assert acc(sh, ctypes.byref(w), base + 2 * 65536, 16, base, None) == 3
    assert acc(sh, ctypes.byref(w), base + 2 * 65536 + 16, 1 << 30, base, None) == 4
    assert acc(sh, ctypes.byref(w), base + 2 * 65536, 1 << 30, base + 2, None) == 4
    st = acc(sh, ctypes.byref(w), base + 2 * 65536, 1 << 30, base + 2 * 65536 + 4096, None)
    assert st == 1 and "overlap" in lib.w8a8_last_error().decode()
    assert acc(ctypes.byref(_shape(0, 128, 8, 2, 256)), None, None, 0, None, None) == 0
    # the allocation-free entry point: a layer whose workspace exceeds the static
    # scratch is refused before any device call
    big = ctypes.byref(_shape(8192, 4096, 64, 2, 1536))
    st = lib.w8a8_moe_forward_static(big, ctypes.byref(w), base, base + 65536, None)
    assert st == 3 and "static scratch" in lib.w8a8_last_error().decode()
    assert lib.w8a8_moe_forward_static(ctypes.byref(_shape(0, 128, 8, 2, 256)), None, None, None, None) == 0
    lay = _lib.MoeLayout()
    assert lib.w8a8_moe_workspace_query(ctypes.byref(_shape(64, 4096, 64, 2, 1536)), ctypes.byref(lay)) == 0
    assert lay.total_bytes <= _lib.STATIC_WORKSPACE_BYTES  # the decode layer fits


def test_gemm_and_quant_argument_checks():
    base = 1 << 40
    assert lib.w8a8_gemm(base, base, base, base, 256, 200, 256, base, None) == 2   # N % 128
    assert lib.w8a8_gemm(base, base, base, base, 256, 256, 100, base, None) == 2   # K % 128
    assert lib.w8a8_gemm(base, base, base, base, 256, 256, 1 << 18, base, None) == 2  # K > 2^17
    assert lib.w8a8_gemm(base, base, base, base, -1, 256, 256, base, None) == 1
    assert lib.w8a8_gemm(base + 1, base, base, base, 256, 256, 256, base, None) == 4
    assert lib.w8a8_gemm(None, None, None, None, 0, 256, 256, None, None) == 0      # M = 0 no-op
    assert lib.w8a8_gemm_i32(base, None, 256, 256, 256, base, None) == 1
    assert lib.w8a8_quantize_rows(base, 4, 0, 0, base, base, None) == 2            # cols = 0
    assert lib.w8a8_quantize_rows(base, 4, 16, 8, base, base, None) == 1           # ld < cols
    assert lib.w8a8_quantize_rows(None, 0, 16, 16, None, None, None) == 0          # rows = 0
    assert lib.w8a8_quantize_rows(base + 2, 4, 16, 16, base, base, None) == 4
    assert lib.w8a8_quantize_rows(base, (1 << 24) + 1, 16, 16, base, base, None) == 2  # rows > 2^24
    assert lib.w8a8_quantize_rows_ex(base, 1 << 40, 16, 16, None, 0, 0.0, 0, base, base, None) == 2
    # scale options: unknown mode, missing or non-finite bound, unknown code, misaligned factor
    assert lib.w8a8_quantize_rows_ex(base, 4, 16, 16, None, 3, 1.0, 0, base, base, None) == 1
    assert lib.w8a8_quantize_rows_ex(base, 4, 16, 16, None, 1, 0.0, 0, base, base, None) == 1
    assert lib.w8a8_quantize_rows_ex(base, 4, 16, 16, None, 2, float("inf"), 0, base, base, None) == 1
    assert lib.w8a8_quantize_rows_ex(base, 4, 16, 16, None, 2, float("nan"), 0, base, base, None) == 1
    assert lib.w8a8_quantize_rows_ex(base, 4, 16, 16, None, 0, 0.0, 5, base, base, None) == 1
    assert lib.w8a8_quantize_rows_ex(base, 4, 16, 16, base + 2, 0, 0.0, 0, base, base, None) == 4
    assert lib.w8a8_quantize_rows_ex(None, 0, 16, 16, None, 1, 2.0, 1, None, None, None) == 0
    assert lib.w8a8_quantize_rows_ex(None, 0, 16, 16, None, 1, 2.0, 2, None, None, None) == 0   # FP8 fast
    assert lib.w8a8_quantize_rows_ex(base, 4, 16, 16, None, 0, 0.0, 3, base, base, None) == 1
    # the FP8 GEMMs share the INT8 GEMM's checks
    for fn in (lib.w8a8_gemm_fp8, lib.w8a8_gemm_fp8_fast):
        assert fn(base, base, base, base, 256, 200, 256, base, None) == 2
        assert fn(base + 1, base, base, base, 256, 256, 256, base, None) == 4
        assert fn(None, None, None, None, 0, 256, 256, None, None) == 0
    # the reciprocal flag needs a factor, and combines with a valid mode only
    assert lib.w8a8_quantize_rows_ex(base, 4, 16, 16, None, 0x10, 0.0, 0, base, base, None) == 1
    assert lib.w8a8_quantize_rows_ex(base, 4, 16, 16, base, 0x13, 1.0, 0, base, base, None) == 1
    assert lib.w8a8_quantize_rows_ex(None, 0, 16, 16, base, 0x10, 0.0, 0, None, None, None) == 0


def test_fused_entry_point_checks():
    """The single-launch layer: T above 64 is refused, and the multi-launch
    layer's argument checks apply, all before any launch."""
    base = 1 << 40
    fused = lib.w8a8_moe_forward_fused
    w = _lib.MoeWeights(base, None, base, base, base, base)
    big = ctypes.byref(_shape(65, 128, 8, 2, 256))
    assert fused(big, ctypes.byref(w), base, base + 65536, base + 2 * 65536, 1 << 30, None) == 2
    assert "64" in lib.w8a8_last_error().decode()
    sh = ctypes.byref(_shape(16, 128, 8, 2, 256))
    assert fused(sh, ctypes.byref(w), None, None, None, 0, None) == 1            # NULL pointers
    assert fused(sh, ctypes.byref(w), base, base + 65536, base + 2 * 65536, 16, None) == 3  # workspace
    assert fused(sh, ctypes.byref(w), base + 4, base + 65536, base + 2 * 65536, 1 << 30, None) == 4
    st = fused(sh, ctypes.byref(w), base, base + 4096, base + 2 * 65536, 1 << 30, None)
    assert st == 1 and "overlap" in lib.w8a8_last_error().decode()
    assert fused(ctypes.byref(_shape(0, 128, 8, 2, 256)), None, None, None, None, 0, None) == 0
    assert fused(ctypes.byref(_shape(16, 100, 8, 2, 256)), ctypes.byref(w), base, base + 65536,
                 base + 2 * 65536, 1 << 30, None) == 2                            # H % 128


def test_pack_size():
    n = ctypes.c_size_t()
    assert lib.w8a8_pack_weights_size(3, 64, 128, _lib.PACK_PLAIN, ctypes.byref(n)) == 0
    assert n.value == 3 * 64 * 128
    assert lib.w8a8_pack_weights_size(1, 64, 100, _lib.PACK_PLAIN, ctypes.byref(n)) == 2
    assert lib.w8a8_pack_weights_size(1, 48, 128, _lib.PACK_GATE_UP, ctypes.byref(n)) == 2
    assert lib.w8a8_pack_weights_size(1, 48, 128, _lib.PACK_PLAIN, ctypes.byref(n)) == 0
    assert lib.w8a8_pack_weights_size(1, 64, 128, 7, ctypes.byref(n)) == 1
    assert lib.w8a8_pack_weights_size(1, 64, 128, 0, None) == 1
    base = 1 << 40
    assert lib.w8a8_pack_weights(base, 1, 64, 128, 0, base, None) == 1   # in place


def test_binding_shares_one_hip_runtime():
    # importing the binding first (before anything imports torch) must still map
    # a single HIP runtime: the library binds to the copy PyTorch loads
    code = ("import re, sys; sys.path.insert(0, %r); import w8a8_quantized_moe_amd; "
            "m = open('/proc/self/maps').read(); "
            "print(len(set(re.findall(r'\\S*libamdhip64\\S*', m))))" % ROOT)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert res.stdout.strip() == "1", res.stdout + res.stderr


# ---------------------------------------------------------------- binding checks
# The C ABI receives bare pointers, so the binding checks every tensor's dtype,
# shape (or byte count) and device before any call: these run on the host,
# with host tensors, and must raise before anything reaches the library.
import torch  # noqa: E402

from w8a8_quantized_moe_amd import api  # noqa: E402


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_binding_rejects_bad_gemm_arguments():
    M, N, K = 4, 128, 128
    a = torch.zeros(M, K, dtype=torch.int8)
    b = torch.zeros(N * K, dtype=torch.int8)
    sa = torch.zeros(M)
    sb = torch.zeros(N)
    _raises(lambda: api.gemm(torch.zeros(M, K + 64, dtype=torch.int8), sa, b, sb, N, K), "a_q must have shape")
    _raises(lambda: api.gemm(a, sa, torch.zeros(N * K - 16, dtype=torch.int8), sb, N, K), "b_packed must hold")
    _raises(lambda: api.gemm(a, torch.zeros(M + 1), b, sb, N, K), "s_a must have shape")
    _raises(lambda: api.gemm(a, sa, b, torch.zeros(N // 2), N, K), "s_b must have shape")
    _raises(lambda: api.gemm(a, sa, b, sb, N, K, out=torch.zeros(M, N - 1)), "out must have shape")
    _raises(lambda: api.gemm(a, sa, b, sb, N, K, out=torch.zeros(M, N, dtype=torch.float16)), "out must be")
    _raises(lambda: api.gemm(a, sa, b, sb, N, K, out=torch.zeros(M, N)), "GPU tensor")
    _raises(lambda: api.gemm_i32(a, b, N, K, out=torch.zeros(M, N)), "out must be torch.int32")
    _raises(lambda: api.gemm_i32(a.float(), b, N, K), "a_q must be torch.int8")
    _raises(lambda: api.gemm_i32(a, b, N, K), "GPU tensor")


def test_binding_rejects_bad_quantize_arguments():
    x = torch.zeros(3, 8)
    _raises(lambda: api.quantize_rows(x), "GPU tensor")
    _raises(lambda: api.quantize_rows(x.t()), "unit column stride")
    _raises(lambda: api.quantize_rows(x.double()), "fp32")


def _weights(E=4, H=128, I=128, **over):
    f = dict(router_w=torch.zeros(E, H), router_b=None, w_gate_up=torch.zeros(E * 2 * I * H, dtype=torch.int8),
             s_gate_up=torch.zeros(E, 2 * I), w_down=torch.zeros(E * H * I, dtype=torch.int8),
             s_down=torch.zeros(E, H))
    f.update(over)
    return api.MoEWeights(E, H, I, **f)


def test_binding_rejects_bad_moe_arguments():
    T, H = 5, 128
    x = torch.zeros(T, H)
    _raises(lambda: api.moe_forward(torch.zeros(T, H + 128), _weights(), 2), "x must have shape")
    _raises(lambda: api.moe_forward(x, _weights(router_w=torch.zeros(4, 64)), 2), "router_w must have shape")
    _raises(lambda: api.moe_forward(x, _weights(router_b=torch.zeros(5)), 2), "router_b must have shape")
    _raises(lambda: api.moe_forward(x, _weights(w_gate_up=torch.zeros(100, dtype=torch.int8)), 2),
            "w_gate_up must hold")
    _raises(lambda: api.moe_forward(x, _weights(s_down=torch.zeros(4, 64)), 2), "s_down must have shape")
    _raises(lambda: api.moe_forward(x, _weights(x_smooth=torch.zeros(64)), 2), "x_smooth must have shape")
    _raises(lambda: api.moe_forward(x, _weights(), 2), "GPU tensor")


def test_binding_rejects_bad_moe_outputs():
    T, H = 5, 128
    x = torch.zeros(T, H)
    w = _weights()
    _raises(lambda: api.moe_forward(x, w, 2, y=torch.zeros(T, H - 1)), "y must have shape")
    _raises(lambda: api.moe_forward(x, w, 2, y=torch.zeros(T, H, dtype=torch.float64)), "y must be")
    _raises(lambda: api.moe_forward(x, w, 2, y=torch.zeros(T, H).t()), "y must have shape")
    _raises(lambda: api.moe_forward(x, w, 2, workspace=torch.zeros(10)), "workspace must be torch.uint8")
    _raises(lambda: api.moe_forward(x, w, 2, y=torch.zeros(T, H), workspace=torch.zeros(10, dtype=torch.uint8)),
            "x must be a GPU tensor")


def test_static_scratch_size_matches_header():
    m = re.search(r"#define\s+W8A8_STATIC_WORKSPACE_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.STATIC_WORKSPACE_BYTES
