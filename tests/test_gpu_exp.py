"""The GEMM epilogues' SiLU on the GPU, over every fp32 input: the library's
device function silu_f32(g) must equal g / (1 + exp_f32_rn(-g)), where
exp_f32_rn is the correctly rounded exponential that the host test ties to
the oracle's (float)exp((double)x) (tests/test_exp_f32_cpu.py).  Together
they make the kernels' SiLU equal the oracle's on all 2^32 inputs, which is
why h is compared bit for bit on every row.  The sweep runs in the tests'
helper library (tests/silu_check.hip, built by build())."""
import ctypes
import os

import pytest

HELPER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "libsilu_check.so")


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()


@pytest.mark.gpu
def test_silu_equals_correctly_rounded_reference_on_every_input(gpu):
    if not os.path.exists(HELPER):
        pytest.fail(f"{HELPER} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(HELPER)
    lib.silu_check_all.restype = ctypes.c_int
    lib.silu_check_all.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.POINTER(ctypes.c_uint32),
                                   ctypes.c_int]
    n = ctypes.c_ulonglong(0)
    ex = (ctypes.c_uint32 * 16)()
    print("silu sweep over 2^32 fp32 inputs", flush=True)
    assert lib.silu_check_all(ctypes.byref(n), ex, 16) == 0
    assert n.value == 0, f"{n.value} inputs differ, e.g. {[hex(v) for v in ex[:min(16, n.value)]]}"
