"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side validation behaves as include/eqlinear.h states.  No call here
reaches a HIP runtime function (no GPU needed)."""
import ctypes
import os
import re

import pytest

import group_dft_structured_amd as eq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("eqlinear.h", "eqconv.h")]


def _lib():
    if not os.path.exists(eq.LIB_PATH):
        pytest.skip("libeqlinear.so not built (run __graft_entry__.build())")
    return eq.load_library()


def declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names |= set(re.findall(r"\b(eq(?:linear|conv)_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary_calls():
    names = declared_functions()
    for n in ("eqlinear_plan_create", "eqlinear_set_weight", "eqlinear_forward",
              "eqlinear_backward_input", "eqlinear_backward_weight", "eqconv_plan_create",
              "eqconv_set_weight", "eqconv_forward", "eqconv_backward_input",
              "eqconv_backward_weight"):
        assert n in names
    assert sorted(eq.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def _raw_plan(lib, C=8, D=8, T=4, dtype=eq.EQL_F32):
    h = ctypes.c_void_p()
    st = lib.eqlinear_plan_create(C, D, T, dtype, ctypes.byref(h))
    return st, h.value


def test_plan_create_validation():
    lib = _lib()
    for T in (-4, 0, 1, 17, 32):                # EQL_ERR_UNSUPPORTED: cyclic groups C_2 .. C_16
        assert _raw_plan(lib, T=T)[0] == 2
    for T in (2, 3, 8, 16):
        st, h = _raw_plan(lib, T=T)
        assert st == 0 and h
        assert lib.eqlinear_plan_destroy(h) == 0
    assert _raw_plan(lib, dtype=7)[0] == 2
    assert _raw_plan(lib, C=0)[0] == 1          # EQL_ERR_INVALID_ARG
    assert _raw_plan(lib, D=-3)[0] == 1
    assert _raw_plan(lib, C=1 << 20)[0] == 1
    assert lib.eqlinear_plan_create(8, 8, 4, 0, None) == 1
    st, h = _raw_plan(lib)
    assert st == 0 and h
    assert lib.eqlinear_plan_destroy(h) == 0
    assert lib.eqlinear_plan_destroy(None) == 0


def test_calls_before_set_weight_and_bad_arguments():
    lib = _lib()
    st, h = _raw_plan(lib, 96, 384, 4, eq.EQL_F16)
    assert st == 0
    try:
        fake = 0x10000  # never dereferenced: every case below fails validation first
        assert lib.eqlinear_forward(h, fake, fake, 16, None) == 3        # NO_WEIGHT
        assert lib.eqlinear_backward_input(h, fake, fake, 16, None) == 3
        assert lib.eqlinear_forward(h, fake, fake, -1, None) == 1
        assert lib.eqlinear_forward(None, fake, fake, 16, None) == 1
        assert lib.eqlinear_set_weight(h, None, None, None) == 1
        assert lib.eqlinear_set_weight(h, fake + 2, None, None) == 4      # MISALIGNED
        assert lib.eqlinear_set_weight(h, fake, fake + 8, None) == 4
        need = lib.eqlinear_backward_weight_workspace(h, 12608)
        assert need > 0
        assert lib.eqlinear_backward_weight_workspace(h, -1) == 0
        assert lib.eqlinear_backward_weight_workspace(None, 10) == 0
        bw = lib.eqlinear_backward_weight
        assert bw(h, fake, fake, None, None, 16, fake, need, None) == 1   # dW NULL
        assert bw(h, None, fake, fake, None, 16, fake, need, None) == 1
        assert bw(h, fake, fake, fake, None, -5, fake, need, None) == 1
        assert bw(h, fake + 4, fake, fake, None, 16, fake, need, None) == 4
        assert bw(h, fake, fake, fake, fake + 4, 16, fake, need, None) == 4
        need16 = lib.eqlinear_backward_weight_workspace(h, 16)
        assert bw(h, fake, fake, fake, None, 16, None, need16, None) == 5  # WORKSPACE
        assert bw(h, fake, fake, fake, None, 16, fake, need16 - 1, None) == 5
    finally:
        lib.eqlinear_plan_destroy(h)


def test_forward_act_rejects_unknown_activation():
    lib = _lib()
    st, h = _raw_plan(lib)
    try:
        # checked before anything else, including the missing weight
        assert lib.eqlinear_forward_act(h, None, None, 0, 3, None) == 1
        assert lib.eqlinear_forward_act(h, None, None, 0, -1, None) == 1
        assert lib.eqlinear_forward_act(h, None, None, 0, 1, None) == 3   # EQL_ERR_NO_WEIGHT
    finally:
        lib.eqlinear_plan_destroy(h)


def test_mac_counts_and_ratio():
    _lib()
    p = eq.eqlinear_plan_create(96, 384, 4, eq.EQL_F16)
    try:
        s, d = eq.eqlinear_mac_counts(p, 12608)
        assert s == 6 * 12608 * 96 * 384 and d == 16 * 12608 * 96 * 384
        assert s * 8 == d * 3   # 2(T-1)/T^2 at T = 4
    finally:
        eq.eqlinear_plan_destroy(p)


def test_mac_counts_every_group_size():
    # Kept frequencies of a real DFT of length T are those numpy's rfft
    # returns; frequency 0 (and T/2 for even T) is real and costs one real
    # product per (n, c, d), every other kept frequency is complex and costs
    # four.  The unrolled dense weight costs T^2.
    import numpy as np
    _lib()
    for T in range(2, 17):
        kept = np.fft.rfft(np.zeros(T)).shape[0]
        real = 1 + (T % 2 == 0)
        products = real + 4 * (kept - real)
        p = eq.eqlinear_plan_create(5, 7, T, eq.EQL_F32)
        try:
            s, d = eq.eqlinear_mac_counts(p, 3)
            assert s == products * 3 * 5 * 7 and d == T * T * 3 * 5 * 7
            # about 2/T of the dense count, exactly 2(T-1)/T^2 for even T
            assert 2 * T - 2 <= products <= 2 * T - 1
            if T % 2 == 0:
                assert s * T * T == d * 2 * (T - 1)
        finally:
            eq.eqlinear_plan_destroy(p)


def test_status_strings_and_python_errors():
    _lib()
    for code in range(8):
        assert eq.eqlinear_status_string(code)
    with pytest.raises(eq.EqlinearError) as ei:
        eq.eqlinear_plan_create(8, 8, 17, eq.EQL_F32)
    assert ei.value.name == "EQL_ERR_UNSUPPORTED"


def test_workspace_grows_with_rows():
    _lib()
    p = eq.eqlinear_plan_create(96, 384, 4, eq.EQL_F16)
    try:
        sizes = [eq.eqlinear_backward_weight_workspace(p, n) for n in (0, 1, 600, 12608)]
        assert sizes[0] == 0 and 0 < sizes[1] <= sizes[2] <= sizes[3]
    finally:
        eq.eqlinear_plan_destroy(p)
    for T in (3, 8, 16):
        p = eq.eqlinear_plan_create(48, 192, T, eq.EQL_F16)
        try:
            sizes = [eq.eqlinear_backward_weight_workspace(p, n) for n in (0, 1, 600, 12608)]
            assert sizes[0] == 0 and 0 < sizes[1] <= sizes[2] <= sizes[3]
        finally:
            eq.eqlinear_plan_destroy(p)


def _raw_group_plan(lib, group, n, C=8, D=8, dtype=eq.EQL_F32):
    h = ctypes.c_void_p()
    st = lib.eqlinear_plan_create_group(C, D, group, n, dtype, ctypes.byref(h))
    return st, h.value


def test_plan_create_group_validation():
    lib = _lib()
    for n in (-1, 0, 1, 9, 16):                 # EQL_ERR_UNSUPPORTED: dihedral D_2 .. D_8
        assert _raw_group_plan(lib, eq.EQL_GROUP_DIHEDRAL, n)[0] == 2
    for n in (2, 3, 4, 8):
        st, h = _raw_group_plan(lib, eq.EQL_GROUP_DIHEDRAL, n)
        assert st == 0 and h
        assert lib.eqlinear_plan_destroy(h) == 0
    st, h = _raw_group_plan(lib, eq.EQL_GROUP_CYCLIC, 16)   # the cyclic group through the same call
    assert st == 0 and h
    assert lib.eqlinear_plan_destroy(h) == 0
    assert _raw_group_plan(lib, eq.EQL_GROUP_CYCLIC, 17)[0] == 2
    assert _raw_group_plan(lib, 5, 4)[0] == 2          # unknown group
    assert _raw_group_plan(lib, eq.EQL_GROUP_DIHEDRAL, 4, dtype=3)[0] == 2
    assert _raw_group_plan(lib, eq.EQL_GROUP_DIHEDRAL, 4, C=0)[0] == 1
    assert lib.eqlinear_plan_create_group(8, 8, eq.EQL_GROUP_DIHEDRAL, 4, 0, None) == 1


def test_mac_counts_dihedral():
    # D_n's real irreducible representations: the one-dimensional ones are
    # the sign patterns a^r b^m (a = -1 needs n even), and the rest of the
    # group order 2n = sum of dim^2 is made of two-dimensional ones; a
    # dim x dim block product costs dim^3 real products per (n, c, d).
    _lib()
    for n in range(2, 9):
        one = 4 if n % 2 == 0 else 2
        two = (2 * n - one) // 4
        assert one + 4 * two == 2 * n
        p = eq.eqlinear_plan_create_group(5, 7, eq.EQL_GROUP_DIHEDRAL, n, eq.EQL_F16)
        try:
            s, d = eq.eqlinear_mac_counts(p, 3)
            assert s == (one + 8 * two) * 3 * 5 * 7 and d == 4 * n * n * 3 * 5 * 7, n
        finally:
            eq.eqlinear_plan_destroy(p)
    p = eq.eqlinear_plan_create_group(96, 384, eq.EQL_GROUP_DIHEDRAL, 4, eq.EQL_F32)
    try:
        s, d = eq.eqlinear_mac_counts(p, 10)
        assert s * 64 == d * 12        # p4m through the group Fourier transform: 12 of 64
    finally:
        eq.eqlinear_plan_destroy(p)


def test_p4m_pairs_dispatch(monkeypatch):
    # binary16 p4m at widths the p4 producer/consumer kernels take runs as p4
    # on paired channels (2C -> 2D): 6 products per paired channel pair,
    # 24 per (c, d); EQL_P4M_PAIRS=0 keeps the group Fourier transform (12)
    _lib()
    for C, paired in ((48, True), (96, True), (16, True), (192, True), (40, False), (5, False), (160, False)):
        p = eq.eqlinear_plan_create_group(C, 64, eq.EQL_GROUP_DIHEDRAL, 4, eq.EQL_F16)
        try:
            s, d = eq.eqlinear_mac_counts(p, 1)
            assert s == (24 if paired else 12) * C * 64 and d == 64 * C * 64, C
            assert eq.eqlinear_backward_weight_workspace(p, 0) == 0
            assert eq.eqlinear_backward_weight_workspace(p, 1000) > 0
        finally:
            eq.eqlinear_plan_destroy(p)
    monkeypatch.setenv("EQL_P4M_PAIRS", "0")
    p = eq.eqlinear_plan_create_group(48, 64, eq.EQL_GROUP_DIHEDRAL, 4, eq.EQL_F16)
    try:
        assert eq.eqlinear_mac_counts(p, 1)[0] == 12 * 48 * 64
    finally:
        eq.eqlinear_plan_destroy(p)


def test_dihedral_workspace_and_python_plan():
    _lib()
    p = eq.eqlinear_plan_create_group(48, 96, eq.EQL_GROUP_DIHEDRAL, 4, eq.EQL_F16)
    try:
        sizes = [eq.eqlinear_backward_weight_workspace(p, n) for n in (0, 1, 600, 12608)]
        assert sizes[0] == 0 and 0 < sizes[1] <= sizes[2] <= sizes[3]
    finally:
        eq.eqlinear_plan_destroy(p)
    with pytest.raises(ValueError):
        eq.Plan(8, 8, "f16", T=7, group="dihedral")
    pl = eq.Plan(8, 8, "f16", T=8, group="dihedral")
    assert pl.T == 8 and pl.group == "dihedral"
    pl.close()


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """The no-allocation weight gradient checks its workspace need against
    its fixed scratch size on the host, before any HIP call."""
    lib = _lib()
    scratch = 32 << 20
    p = eq.eqlinear_plan_create(2048, 2048, 4, eq.EQL_F16)
    try:
        N = 1 << 16
        assert eq.eqlinear_backward_weight_workspace(p, N) > scratch
        # any aligned non-null addresses: the call returns before using them
        fake = 1 << 20
        st = lib.eqlinear_backward_weight_noalloc(p, fake, fake, fake, fake, N, None)
        assert st == 5                                    # EQL_ERR_WORKSPACE
        assert "scratch" in eq.eqlinear_last_error()
        assert lib.eqlinear_backward_weight_noalloc(p, fake, fake, None, None, 16, None) == 1
        assert lib.eqlinear_backward_weight_noalloc(p, fake + 8, fake, fake, fake, 16, None) == 4
        assert lib.eqlinear_backward_weight_noalloc(None, fake, fake, fake, fake, 16, None) == 1
    finally:
        eq.eqlinear_plan_destroy(p)
