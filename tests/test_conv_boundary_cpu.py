"""Host-side validation of the p4 group-convolution entry points
(include/eqconv.h) on the CPU: no call here reaches a HIP runtime function."""
import ctypes

import pytest

import group_dft_structured_amd as eq
from tests.test_boundary_cpu import _lib

FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _plan(lib, C=8, D=12, k=3, dtype=eq.EQL_F16):
    h = ctypes.c_void_p()
    st = lib.eqconv_plan_create(C, D, k, dtype, ctypes.byref(h))
    return st, h.value


def test_plan_create_validation():
    lib = _lib()
    for k in (0, 2, 4, 9, -1):
        assert _plan(lib, k=k)[0] == 2               # EQL_ERR_UNSUPPORTED
    for C, D in ((6, 8), (8, 10), (1, 4)):
        assert _plan(lib, C=C, D=D)[0] == 2          # channels not multiples of 4
    assert _plan(lib, C=8192, k=3)[0] == 2           # k^2 C above 65536
    assert _plan(lib, dtype=5)[0] == 2
    assert _plan(lib, C=0)[0] == 1 and _plan(lib, D=-4)[0] == 1
    assert lib.eqconv_plan_create(8, 8, 3, 0, None) == 1
    for k in (1, 3, 5, 7):
        st, h = _plan(lib, k=k)
        assert st == 0 and h
        assert lib.eqconv_plan_destroy(h) == 0
    assert lib.eqconv_plan_destroy(None) == 0


def test_calls_validate_before_the_gpu():
    lib = _lib()
    st, h = _plan(lib)
    assert st == 0
    try:
        assert lib.eqconv_forward(h, FAKE, FAKE, 2, 5, 5, 0, None) == 3        # NO_WEIGHT
        assert lib.eqconv_backward_input(h, FAKE, FAKE, 2, 5, 5, None) == 3
        assert lib.eqconv_forward(h, FAKE, FAKE, 2, 5, 5, 3, None) == 1        # bad activation
        assert lib.eqconv_forward(h, FAKE, FAKE, -1, 5, 5, 0, None) == 1
        assert lib.eqconv_forward(h, FAKE, FAKE, 1 << 20, 1 << 10, 1 << 10, 0, None) == 1
        assert lib.eqconv_forward(None, FAKE, FAKE, 2, 5, 5, 0, None) == 1
        assert lib.eqconv_set_weight(h, None, None, None) == 1
        assert lib.eqconv_set_weight(h, FAKE + 2, None, None) == 4             # MISALIGNED
        need = lib.eqconv_backward_weight_workspace(h, 2, 5, 5)
        assert need > 0
        assert lib.eqconv_backward_weight_workspace(h, -1, 5, 5) == 0
        assert lib.eqconv_backward_weight_workspace(None, 2, 5, 5) == 0
        bw = lib.eqconv_backward_weight
        assert bw(h, FAKE, FAKE, None, None, 2, 5, 5, FAKE, need, None) == 1   # dpsi NULL
        assert bw(h, None, FAKE, FAKE, None, 2, 5, 5, FAKE, need, None) == 1
        assert bw(h, FAKE + 4, FAKE, FAKE, None, 2, 5, 5, FAKE, need, None) == 4
        assert bw(h, FAKE, FAKE, FAKE, None, 2, 5, 5, None, need, None) == 5   # WORKSPACE
        assert bw(h, FAKE, FAKE, FAKE, None, 2, 5, 5, FAKE, need - 1, None) == 5
    finally:
        lib.eqconv_plan_destroy(h)


def test_workspace_holds_the_patches():
    lib = _lib()
    for dtype, es in ((eq.EQL_F16, 2), (eq.EQL_F32, 4)):
        st, h = _plan(lib, C=48, D=48, k=3, dtype=dtype)
        try:
            P = 64 * 56 * 56
            need = lib.eqconv_backward_weight_workspace(h, 64, 56, 56)
            assert need >= P * 9 * 48 * 4 * es + 48 * 9 * 48 * 4 * 4
            assert lib.eqconv_backward_weight_workspace(h, 0, 56, 56) > 0   # the gradient fold
        finally:
            lib.eqconv_plan_destroy(h)


def test_mac_counts_are_three_eighths():
    _lib()
    h = eq.eqconv_plan_create(48, 48, 3, eq.EQL_F16)
    try:
        s, d = eq.eqconv_mac_counts(h, 64, 56, 56)
        assert s == 6 * 9 * 48 * 48 * 64 * 56 * 56 and d * 3 == s * 8
    finally:
        eq.eqconv_plan_destroy(h)


def test_python_plan_rejects_wrong_shapes():
    _lib()
    torch = pytest.importorskip("torch")
    p = eq.ConvPlan(8, 12, 3, "f32")
    with pytest.raises(ValueError):
        p.set_weight(torch.zeros((12, 8, 3, 3, 4)))  # a CPU tensor is rejected
    p.close()
