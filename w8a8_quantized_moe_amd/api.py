"""Python binding of the w8a8moe C ABI.  Argument marshalling only: every step
of the computation runs in the HIP kernels of libw8a8moe.so.  PyTorch provides
device memory and the current stream."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import check, lib

__all__ = [
    "quantize_rows", "pack_weights", "gemm", "gemm_i32", "MoEWeights", "moe_workspace_layout",
    "moe_forward", "moe_forward_fused", "moe_forward_static", "moe_gate_up_acc", "workspace_views",
]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, dtype, name, shape=None, numel=None, gpu=True):
    """Reject a tensor the C ABI cannot size-check: wrong type, dtype, shape or
    element count, non-contiguous, or (gpu) not in GPU memory (the library
    would read or write past it on the device)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    dtypes = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(map(str, dtypes))}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if gpu and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _check_all(*specs):
    """specs: (tensor, dtype, name[, shape[, numel]]) each.  Every dtype and
    shape is checked before any device, so a host without a GPU still
    reaches (and tests) every shape check."""
    for sp in specs:
        t, dtype, name = sp[:3]
        _dev(t, dtype, name, sp[3] if len(sp) > 3 else None, sp[4] if len(sp) > 4 else None, gpu=False)
    for sp in specs:
        if not sp[0].is_cuda:
            raise ValueError(f"{sp[2]} must be a GPU tensor")
    _check_device(*[(sp[0], sp[2]) for sp in specs])


def _check_device(*named):
    """The library runs on the current device's current stream: every tensor
    (name pairs; None skipped) must live on that device."""
    dev = None
    for t, name in named:
        if t is None:
            continue
        if dev is None:
            dev = torch.cuda.current_device()
        if t.device.index != dev:
            raise ValueError(f"{name} is on {t.device}, the current device is cuda:{dev}")


def quantize_rows(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                  scale: Optional[torch.Tensor] = None, code: int = _lib.CODE_INT8,
                  col_mul: Optional[torch.Tensor] = None, scale_mode: int = _lib.SCALE_DYNAMIC,
                  clip: float = 0.0, col_reciprocal: bool = False):
    """Per-row quantisation of a [rows, cols] fp32 matrix (any leading
    dimension via stride(0)) to int8 codes or (code=CODE_FP8 or CODE_FP8_FAST,
    which store the same codes) uint8 E4M3 codes,
    optionally with a per-column factor col_mul [cols] and a clipped or static
    scale (w8a8_quantize_rows_ex); with col_reciprocal the factor applied is
    1 / col_mul (the library divides).  Returns (q [rows, cols], scale fp32
    [rows])."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D fp32 tensor with unit column stride")
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    rows, cols = x.shape
    if code not in (_lib.CODE_INT8, _lib.CODE_FP8, _lib.CODE_FP8_FAST):
        raise ValueError(f"unknown code {code}")
    fp8 = code != _lib.CODE_INT8
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8 if fp8 else torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check_all((q, torch.uint8 if fp8 else torch.int8, "q", (rows, cols)), (scale, torch.float32, "scale", (rows,)))
    if col_reciprocal and col_mul is None:
        raise ValueError("col_reciprocal needs col_mul")
    if col_mul is not None:
        _dev(col_mul, torch.float32, "col_mul", shape=(cols,))
    _check_device((x, "x"), (col_mul, "col_mul"))
    if col_mul is not None or scale_mode != _lib.SCALE_DYNAMIC:
        if col_mul is not None:
            _dev(col_mul, torch.float32, "col_mul", shape=(cols,))
        mode = scale_mode | (_lib.SCALE_COL_RECIPROCAL if col_reciprocal else 0)
        check(lib.w8a8_quantize_rows_ex(_ptr(x), rows, cols, x.stride(0), _ptr(col_mul), mode,
                                        float(clip), code, _ptr(q), _ptr(scale), _stream()))
        return q, scale
    fn = lib.w8a8_quantize_rows_fp8 if fp8 else lib.w8a8_quantize_rows
    check(fn(_ptr(x), rows, cols, x.stride(0), _ptr(q), _ptr(scale), _stream()))
    return q, scale


def pack_weights(w: torch.Tensor, kind: int = _lib.PACK_PLAIN) -> torch.Tensor:
    """Re-lay int8 weights [groups, n, k] (or [n, k]) into the GEMM tile order."""
    if not isinstance(w, torch.Tensor) or w.dim() not in (2, 3):
        raise ValueError("w must be a [groups, n, k] or [n, k] tensor")
    if w.dim() == 2:
        w = w.unsqueeze(0)
    if w.dtype == torch.uint8:  # FP8 codes: the packing moves bytes
        w = w.view(torch.int8)
    _dev(w, torch.int8, "w")
    _check_device((w, "w"))
    g, n, k = w.shape
    nbytes = ctypes.c_size_t()
    check(lib.w8a8_pack_weights_size(g, n, k, kind, ctypes.byref(nbytes)))
    packed = torch.empty((nbytes.value,), dtype=torch.int8, device=w.device)
    check(lib.w8a8_pack_weights(_ptr(w), g, n, k, kind, _ptr(packed), _stream()))
    return packed


def _gemm_specs(a_q, b_packed, N: int, K: int, a_dtype):
    if not isinstance(a_q, torch.Tensor) or a_q.dim() != 2:
        raise ValueError("a_q must be a 2-D tensor [M, K]")
    M = a_q.shape[0]
    return M, [(a_q, a_dtype, "a_q", (M, K)), (b_packed, (torch.int8, torch.uint8), "b_packed", None, N * K)]


def gemm(a_q, s_a, b_packed, s_b, N: int, K: int, out=None, fp8_fast: bool = False) -> torch.Tensor:
    """Dense W8A8 GEMM: out = ((float)(a_q @ b^T) * s_a[:, None]) * s_b[None, :].
    int8 a_q: int8 codes (exact int32 accumulation); uint8 a_q: FP8 E4M3 codes
    (exact products summed in fp32; with fp8_fast on the FP8 matrix cores),
    with b packed from codes of the same kind.
    a_q [M, K]; b_packed: N*K bytes from pack_weights; s_a [M]; s_b [N];
    out [M, N] fp32 (allocated if None)."""
    fp8 = isinstance(a_q, torch.Tensor) and a_q.dtype == torch.uint8
    M, specs = _gemm_specs(a_q, b_packed, N, K, torch.uint8 if fp8 else torch.int8)
    specs += [(s_a, torch.float32, "s_a", (M,)), (s_b, torch.float32, "s_b", (N,))]
    if out is not None:
        specs.append((out, torch.float32, "out", (M, N)))
    _check_all(*specs)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_q.device)
    if fp8_fast and not fp8:
        raise ValueError("fp8_fast needs uint8 (E4M3) codes")
    fn = (lib.w8a8_gemm_fp8_fast if fp8_fast else lib.w8a8_gemm_fp8) if fp8 else lib.w8a8_gemm
    check(fn(_ptr(a_q), _ptr(s_a), _ptr(b_packed), _ptr(s_b), M, N, K, _ptr(out), _stream()))
    return out


def gemm_i32(a_q, b_packed, N: int, K: int, out=None) -> torch.Tensor:
    """Raw int32 accumulators a_q @ b^T (for checking); a_q [M, K] int8,
    b_packed N*K bytes, out [M, N] int32 (allocated if None)."""
    M, specs = _gemm_specs(a_q, b_packed, N, K, torch.int8)
    if out is not None:
        specs.append((out, torch.int32, "out", (M, N)))
    _check_all(*specs)
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=a_q.device)
    check(lib.w8a8_gemm_i32(_ptr(a_q), _ptr(b_packed), M, N, K, _ptr(out), _stream()))
    return out


@dataclass
class MoEWeights:
    """Device-resident weights of one MoE layer in the library's layout."""
    E: int
    H: int
    I: int
    router_w: torch.Tensor            # [E, H] fp32
    router_b: Optional[torch.Tensor]  # [E] fp32 or None
    w_gate_up: torch.Tensor           # packed int8 (GATE_UP) of [E, 2I, H]
    s_gate_up: torch.Tensor           # [E, 2I] fp32
    w_down: torch.Tensor              # packed int8 (PLAIN) of [E, H, I]
    s_down: torch.Tensor              # [E, H] fp32
    code: int = _lib.CODE_INT8        # CODE_INT8, CODE_FP8 or CODE_FP8_FAST (E4M3 codes)
    x_smooth: Optional[torch.Tensor] = None  # [H] fp32 SmoothQuant factor on x, or None
    x_scale_mode: int = _lib.SCALE_DYNAMIC   # scale of x: dynamic, clipped or static
    x_clip: float = 0.0                      # the bound of the clipped / static modes

    @classmethod
    def from_int8(cls, router_w, router_b, w_gu, s_gu, w_d, s_d, x_smooth=None,
                  x_scale_mode: int = _lib.SCALE_DYNAMIC, x_clip: float = 0.0, fp8_fast: bool = False):
        """From int8 codes [E, 2I, H] / [E, H, I] with per-output-channel scales
        (uint8 tensors: FP8 E4M3 codes, and the layer runs with FP8 codes --
        exact products summed in fp32, or with fp8_fast on the FP8 matrix
        cores).  With x_smooth the gate-up codes must already carry 1/x_smooth
        on their input channels."""
        E, twoI, H = w_gu.shape
        if w_gu.dtype == torch.uint8:
            code = _lib.CODE_FP8_FAST if fp8_fast else _lib.CODE_FP8
        elif fp8_fast:
            raise ValueError("fp8_fast needs uint8 (E4M3) codes")
        else:
            code = _lib.CODE_INT8
        return cls(E, H, twoI // 2, router_w.contiguous(),
                   None if router_b is None else router_b.contiguous(),
                   pack_weights(w_gu.contiguous(), _lib.PACK_GATE_UP), s_gu.contiguous(),
                   pack_weights(w_d.contiguous(), _lib.PACK_PLAIN), s_d.contiguous(), code,
                   None if x_smooth is None else x_smooth.contiguous(), x_scale_mode, float(x_clip))

    @classmethod
    def from_fp32(cls, router_w, router_b, w_gu_f32, w_d_f32, keep_codes=False,
                  code: int = _lib.CODE_INT8, x_smooth=None, x_scale_mode: int = _lib.SCALE_DYNAMIC,
                  x_clip: float = 0.0):
        """Quantise fp32 expert weights per output channel with the library's
        row quantiser (offline step), then pack.  With x_smooth (SmoothQuant)
        the gate-up weights are quantised with 1/x_smooth on their input
        channels (the library takes the reciprocal).  With keep_codes the unpacked codes and scales are returned
        as well."""
        E, twoI, H = w_gu_f32.shape
        I = twoI // 2
        sm = None if x_smooth is None else x_smooth.contiguous()
        q_gu, s_gu = quantize_rows(w_gu_f32.reshape(E * twoI, H).contiguous(), code=code, col_mul=sm,
                                   col_reciprocal=sm is not None)
        q_d, s_d = quantize_rows(w_d_f32.reshape(E * H, I).contiguous(), code=code)
        q_gu = q_gu.view(E, twoI, H)
        q_d = q_d.view(E, H, I)
        w = cls.from_int8(router_w, router_b, q_gu, s_gu.view(E, twoI), q_d, s_d.view(E, H),
                          x_smooth, x_scale_mode, x_clip, fp8_fast=code == _lib.CODE_FP8_FAST)
        if keep_codes:
            return w, dict(w_gu=q_gu, s_gu=s_gu.view(E, twoI), w_d=q_d, s_d=s_d.view(E, H))
        return w

    def specs(self) -> list:
        """dtype, shape (packed weights: byte count) and name of every tensor,
        for the binding's checks: the C ABI receives bare pointers and cannot
        size-check them."""
        E, H, I = self.E, self.H, self.I
        sp = [(self.router_w, torch.float32, "router_w", (E, H))]
        if self.router_b is not None:
            sp.append((self.router_b, torch.float32, "router_b", (E,)))
        sp += [(self.w_gate_up, (torch.int8, torch.uint8), "w_gate_up", None, E * 2 * I * H),
               (self.s_gate_up, torch.float32, "s_gate_up", (E, 2 * I)),
               (self.w_down, (torch.int8, torch.uint8), "w_down", None, E * H * I),
               (self.s_down, torch.float32, "s_down", (E, H))]
        if self.x_smooth is not None:
            sp.append((self.x_smooth, torch.float32, "x_smooth", (H,)))
        return sp

    def _struct(self):
        return _lib.MoeWeights(self.router_w.data_ptr(),
                               None if self.router_b is None else self.router_b.data_ptr(),
                               self.w_gate_up.data_ptr(), self.s_gate_up.data_ptr(),
                               self.w_down.data_ptr(), self.s_down.data_ptr(), self.code,
                               None if self.x_smooth is None else self.x_smooth.data_ptr(),
                               self.x_scale_mode, self.x_clip)


def _shape(T, H, E, k, I):
    return _lib.MoeShape(T, H, E, k, I)


def moe_workspace_layout(T: int, H: int, E: int, top_k: int, I: int) -> dict:
    lay = _lib.MoeLayout()
    sh = _shape(T, H, E, top_k, I)
    check(lib.w8a8_moe_workspace_query(ctypes.byref(sh), ctypes.byref(lay)))
    return {f: int(getattr(lay, f)) for f in _lib.LAYOUT_FIELDS}


def moe_forward(x: torch.Tensor, weights: MoEWeights, top_k: int, y: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, events=None) -> torch.Tensor:
    """y = MoE expert layer(x), x [T, H] fp32 on the GPU.  ``workspace`` is a
    uint8 GPU tensor of at least moe_workspace_layout(...)['total_bytes']
    (allocated here if None); it holds the intermediates afterwards.
    ``events``: optional ctypes array of len(MOE_STAGES)+1 hipEvent_t handles
    recorded at the stage boundaries (see w8a8_moe_forward_events)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [T, H]")
    T, H = x.shape
    specs = [(x, torch.float32, "x", (T, weights.H))] + weights.specs()
    if y is not None:
        specs.append((y, torch.float32, "y", (T, H)))
    if workspace is not None:
        specs.append((workspace, torch.uint8, "workspace"))
    _check_all(*specs)
    lay = moe_workspace_layout(T, H, weights.E, top_k, weights.I)
    if T > 0 and workspace is not None and workspace.numel() < lay["total_bytes"]:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the layer needs {lay['total_bytes']}")
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty((max(lay["total_bytes"], 256),), dtype=torch.uint8, device=x.device)
    sh = _shape(T, H, weights.E, top_k, weights.I)
    wts = weights._struct()
    if events is None:
        check(lib.w8a8_moe_forward(ctypes.byref(sh), ctypes.byref(wts), _ptr(x), _ptr(y),
                                   _ptr(workspace), workspace.numel(), _stream()))
    else:
        check(lib.w8a8_moe_forward_events(ctypes.byref(sh), ctypes.byref(wts), _ptr(x), _ptr(y),
                                          _ptr(workspace), workspace.numel(), events, _stream()))
    return y


def moe_forward_fused(x: torch.Tensor, weights: MoEWeights, top_k: int, y: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer of a decode-sized batch (T <= 64) in one persistent launch
    (w8a8_moe_forward_fused); arguments and the workspace as for moe_forward."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [T, H]")
    T, H = x.shape
    specs = [(x, torch.float32, "x", (T, weights.H))] + weights.specs()
    if y is not None:
        specs.append((y, torch.float32, "y", (T, H)))
    if workspace is not None:
        specs.append((workspace, torch.uint8, "workspace"))
    _check_all(*specs)
    lay = moe_workspace_layout(T, H, weights.E, top_k, weights.I)
    if T > 0 and workspace is not None and workspace.numel() < lay["total_bytes"]:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the layer needs {lay['total_bytes']}")
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty((max(lay["total_bytes"], 256),), dtype=torch.uint8, device=x.device)
    sh = _shape(T, H, weights.E, top_k, weights.I)
    wts = weights._struct()
    check(lib.w8a8_moe_forward_fused(ctypes.byref(sh), ctypes.byref(wts), _ptr(x), _ptr(y), _ptr(workspace),
                                     workspace.numel(), _stream()))
    return y


def moe_forward_static(x: torch.Tensor, weights: MoEWeights, top_k: int,
                       y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer without a workspace (w8a8_moe_forward_static): the library's
    static per-device scratch holds the intermediates, so the call allocates
    nothing on the device (y is allocated here only if None).  Calls that
    overlap on one device race on that scratch."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [T, H]")
    T, H = x.shape
    specs = [(x, torch.float32, "x", (T, weights.H))] + weights.specs()
    if y is not None:
        specs.append((y, torch.float32, "y", (T, H)))
    _check_all(*specs)
    if y is None:
        y = torch.empty_like(x)
    sh = _shape(T, H, weights.E, top_k, weights.I)
    wts = weights._struct()
    check(lib.w8a8_moe_forward_static(ctypes.byref(sh), ctypes.byref(wts), _ptr(x), _ptr(y), _stream()))
    return y


def moe_gate_up_acc(T: int, weights: MoEWeights, top_k: int, workspace: torch.Tensor,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The grouped gate-up GEMM's raw int32 accumulators [T*top_k, 2I] over the
    routing the last moe_forward call left in ``workspace`` (INT8 codes; for
    checking): row r is the r-th expert-sorted row, column c < I gate
    channel c, column I + c up channel c."""
    A, I = T * top_k, weights.I
    specs = weights.specs() + [(workspace, torch.uint8, "workspace")]
    if out is not None:
        specs.append((out, torch.int32, "out", (A, 2 * I)))
    _check_all(*specs)
    if out is None:
        out = torch.empty((A, 2 * I), dtype=torch.int32, device=workspace.device)
    sh = _shape(T, weights.H, weights.E, top_k, I)
    wts = weights._struct()
    check(lib.w8a8_moe_gate_up_acc(ctypes.byref(sh), ctypes.byref(wts), _ptr(workspace), workspace.numel(),
                                   _ptr(out), _stream()))
    return out


def workspace_views(workspace: torch.Tensor, T: int, H: int, E: int, top_k: int, I: int) -> dict:
    """Tensors viewing the intermediates a moe_forward call left in ``workspace``."""
    lay = moe_workspace_layout(T, H, E, top_k, I)
    A = T * top_k

    def view(name, dtype, shape):
        n = 1
        for s in shape:
            n *= s
        esz = torch.empty((), dtype=dtype).element_size()
        off = lay[name]
        return workspace[off:off + n * esz].view(dtype).view(*shape)

    return dict(
        x_q=view("x_q", torch.int8, (T, H)),
        x_scale=view("x_scale", torch.float32, (T,)),
        logits=view("logits", torch.float32, (T, E)),
        topk_ids=view("topk_ids", torch.int32, (T, top_k)),
        topk_w=view("topk_w", torch.float32, (T, top_k)),
        expert_counts=view("expert_counts", torch.int32, (E,)),
        expert_offsets=view("expert_offsets", torch.int32, (E + 1,)),
        sorted_assign=view("sorted_assign", torch.int32, (A,)),
        h=view("h", torch.float32, (A, I)),
        h_q=view("h_q", torch.int8, (A, I)),
        h_scale=view("h_scale", torch.float32, (A,)),
        o=view("o", torch.float32, (A, H)),
    )
