"""Python binding of libeqlinear, the EQ-Linear layer of the cyclic rotation
groups (p4 and C_2 .. C_16) and of the dihedral groups (p4m and D_2 .. D_8),
and the p4 group convolution on the plane, on MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libeqlinear.so``.  PyTorch supplies device memory and streams; the functions
below take torch tensors (or raw integer pointers) and pass their addresses to
the C ABI declared in ``include/eqlinear.h`` and ``include/eqconv.h``, under
the same names.

There is no fallback: if the library is missing, importing the binding's
functions raises ``EqlinearUnavailable`` on first use.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libeqlinear.so")

EQL_F32 = 0
EQL_F16 = 1

EQL_GROUP_CYCLIC = 0
EQL_GROUP_DIHEDRAL = 1
GROUPS = {"cyclic": EQL_GROUP_CYCLIC, "dihedral": EQL_GROUP_DIHEDRAL}

EQL_ACT_NONE = 0
EQL_ACT_GELU = 1
EQL_ACT_GELU_TANH = 2
ACTIVATIONS = {None: EQL_ACT_NONE, "none": EQL_ACT_NONE, "gelu": EQL_ACT_GELU,
               "gelu_tanh": EQL_ACT_GELU_TANH}

STATUS = {
    0: "EQL_OK",
    1: "EQL_ERR_INVALID_ARG",
    2: "EQL_ERR_UNSUPPORTED",
    3: "EQL_ERR_NO_WEIGHT",
    4: "EQL_ERR_MISALIGNED",
    5: "EQL_ERR_WORKSPACE",
    6: "EQL_ERR_ALLOC",
    7: "EQL_ERR_HIP",
}

EXPORTED = (
    "eqlinear_plan_create",
    "eqlinear_plan_create_group",
    "eqlinear_plan_destroy",
    "eqlinear_set_weight",
    "eqlinear_forward",
    "eqlinear_forward_act",
    "eqlinear_backward_input",
    "eqlinear_backward_weight_workspace",
    "eqlinear_backward_weight",
    "eqlinear_backward_weight_noalloc",
    "eqlinear_status_string",
    "eqlinear_last_error",
    "eqlinear_mac_counts",
    "eqconv_plan_create",
    "eqconv_plan_destroy",
    "eqconv_set_weight",
    "eqconv_forward",
    "eqconv_backward_input",
    "eqconv_backward_weight_workspace",
    "eqconv_backward_weight",
    "eqconv_mac_counts",
)


class EqlinearUnavailable(RuntimeError):
    pass


class EqlinearError(RuntimeError):
    def __init__(self, status, where, detail=""):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = f"{where}: {self.name}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


_lib = None


def load_library(path=LIB_PATH):
    """Load libeqlinear.so and declare its signatures (cached)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise EqlinearUnavailable(
            f"{path} is not built; run `python -m group_dft_structured_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.eqlinear_plan_create.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(vp)]
    lib.eqlinear_plan_create.restype = st
    lib.eqlinear_plan_create_group.argtypes = [i64, i64, ctypes.c_int, i64, ctypes.c_int,
                                               ctypes.POINTER(vp)]
    lib.eqlinear_plan_create_group.restype = st
    lib.eqlinear_plan_destroy.argtypes = [vp]
    lib.eqlinear_plan_destroy.restype = st
    lib.eqlinear_set_weight.argtypes = [vp, vp, vp, vp]
    lib.eqlinear_set_weight.restype = st
    lib.eqlinear_forward.argtypes = [vp, vp, vp, i64, vp]
    lib.eqlinear_forward.restype = st
    lib.eqlinear_forward_act.argtypes = [vp, vp, vp, i64, ctypes.c_int, vp]
    lib.eqlinear_forward_act.restype = st
    lib.eqlinear_backward_input.argtypes = [vp, vp, vp, i64, vp]
    lib.eqlinear_backward_input.restype = st
    lib.eqlinear_backward_weight_workspace.argtypes = [vp, i64]
    lib.eqlinear_backward_weight_workspace.restype = ctypes.c_size_t
    lib.eqlinear_backward_weight.argtypes = [vp, vp, vp, vp, vp, i64, vp, ctypes.c_size_t, vp]
    lib.eqlinear_backward_weight.restype = st
    lib.eqlinear_backward_weight_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, vp]
    lib.eqlinear_backward_weight_noalloc.restype = st
    lib.eqlinear_status_string.argtypes = [st]
    lib.eqlinear_status_string.restype = ctypes.c_char_p
    lib.eqlinear_last_error.argtypes = []
    lib.eqlinear_last_error.restype = ctypes.c_char_p
    lib.eqlinear_mac_counts.argtypes = [vp, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.eqlinear_mac_counts.restype = st
    lib.eqconv_plan_create.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(vp)]
    lib.eqconv_plan_create.restype = st
    lib.eqconv_plan_destroy.argtypes = [vp]
    lib.eqconv_plan_destroy.restype = st
    lib.eqconv_set_weight.argtypes = [vp, vp, vp, vp]
    lib.eqconv_set_weight.restype = st
    lib.eqconv_forward.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.eqconv_forward.restype = st
    lib.eqconv_backward_input.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.eqconv_backward_input.restype = st
    lib.eqconv_backward_weight_workspace.argtypes = [vp, i64, i64, i64]
    lib.eqconv_backward_weight_workspace.restype = ctypes.c_size_t
    lib.eqconv_backward_weight.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t,
                                           vp]
    lib.eqconv_backward_weight.restype = st
    lib.eqconv_mac_counts.argtypes = [vp, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.eqconv_mac_counts.restype = st
    _lib = lib
    return lib


def _ptr(t):
    """Address of a torch tensor, a raw int address, or None -> NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != 0:
        lib = load_library()
        detail = lib.eqlinear_last_error().decode()
        raise EqlinearError(status, where, detail)


# --------------------------------------------------------------------------
# C ABI, one function per entry point (same names).

def eqlinear_plan_create(C, D, T=4, dtype=EQL_F32):
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.eqlinear_plan_create(C, D, T, dtype, ctypes.byref(h)), "eqlinear_plan_create")
    return h.value


def eqlinear_plan_create_group(C, D, group, n, dtype=EQL_F32):
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.eqlinear_plan_create_group(C, D, group, n, dtype, ctypes.byref(h)),
           "eqlinear_plan_create_group")
    return h.value


def eqlinear_plan_destroy(plan):
    _check(load_library().eqlinear_plan_destroy(plan), "eqlinear_plan_destroy")


def eqlinear_set_weight(plan, W, bias=None, stream=None):
    _check(load_library().eqlinear_set_weight(plan, _ptr(W), _ptr(bias), _stream(stream)),
           "eqlinear_set_weight")


def eqlinear_forward(plan, x, y, N, stream=None):
    _check(load_library().eqlinear_forward(plan, _ptr(x), _ptr(y), N, _stream(stream)),
           "eqlinear_forward")


def eqlinear_forward_act(plan, x, y, N, act, stream=None):
    _check(load_library().eqlinear_forward_act(plan, _ptr(x), _ptr(y), N, act, _stream(stream)),
           "eqlinear_forward_act")


def eqlinear_backward_input(plan, dy, dx, N, stream=None):
    _check(load_library().eqlinear_backward_input(plan, _ptr(dy), _ptr(dx), N, _stream(stream)),
           "eqlinear_backward_input")


def eqlinear_backward_weight_workspace(plan, N):
    return int(load_library().eqlinear_backward_weight_workspace(plan, N))


def eqlinear_backward_weight(plan, x, dy, dW, dbias, N, workspace, workspace_bytes, stream=None):
    _check(load_library().eqlinear_backward_weight(
        plan, _ptr(x), _ptr(dy), _ptr(dW), _ptr(dbias), N, _ptr(workspace), workspace_bytes,
        _stream(stream)), "eqlinear_backward_weight")


def eqlinear_backward_weight_noalloc(plan, x, dy, dW, dbias, N, stream=None):
    _check(load_library().eqlinear_backward_weight_noalloc(
        plan, _ptr(x), _ptr(dy), _ptr(dW), _ptr(dbias), N, _stream(stream)),
        "eqlinear_backward_weight_noalloc")


def eqlinear_status_string(status):
    return load_library().eqlinear_status_string(status).decode()


def eqlinear_last_error():
    return load_library().eqlinear_last_error().decode()


def eqlinear_mac_counts(plan, N):
    s, d = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().eqlinear_mac_counts(plan, N, ctypes.byref(s), ctypes.byref(d)),
           "eqlinear_mac_counts")
    return s.value, d.value


def eqconv_plan_create(C, D, k, dtype=EQL_F32):
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.eqconv_plan_create(C, D, k, dtype, ctypes.byref(h)), "eqconv_plan_create")
    return h.value


def eqconv_plan_destroy(plan):
    _check(load_library().eqconv_plan_destroy(plan), "eqconv_plan_destroy")


def eqconv_set_weight(plan, psi, bias=None, stream=None):
    _check(load_library().eqconv_set_weight(plan, _ptr(psi), _ptr(bias), _stream(stream)),
           "eqconv_set_weight")


def eqconv_forward(plan, f, y, N, H, W, act=EQL_ACT_NONE, stream=None):
    _check(load_library().eqconv_forward(plan, _ptr(f), _ptr(y), N, H, W, act, _stream(stream)),
           "eqconv_forward")


def eqconv_backward_input(plan, dy, df, N, H, W, stream=None):
    _check(load_library().eqconv_backward_input(plan, _ptr(dy), _ptr(df), N, H, W,
                                                _stream(stream)), "eqconv_backward_input")


def eqconv_backward_weight_workspace(plan, N, H, W):
    return int(load_library().eqconv_backward_weight_workspace(plan, N, H, W))


def eqconv_backward_weight(plan, f, dy, dpsi, dbias, N, H, W, workspace, workspace_bytes,
                           stream=None):
    _check(load_library().eqconv_backward_weight(
        plan, _ptr(f), _ptr(dy), _ptr(dpsi), _ptr(dbias), N, H, W, _ptr(workspace),
        workspace_bytes, _stream(stream)), "eqconv_backward_weight")


def eqconv_mac_counts(plan, N, H, W):
    s, d = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().eqconv_mac_counts(plan, N, H, W, ctypes.byref(s), ctypes.byref(d)),
           "eqconv_mac_counts")
    return s.value, d.value


# --------------------------------------------------------------------------
# Convenience wrapper over torch tensors (still only marshalling).

_DTYPE_CODE = {"f32": EQL_F32, "f16": EQL_F16}


class Plan:
    """Owns one plan handle; calls take contiguous torch CUDA tensors.

    group="cyclic": C_T with T group values per channel (T = 4 is p4).
    group="dihedral": D_n with n = T // 2 rotations and T = 2n group values
    per channel (T = 8 is p4m); T must then be even."""

    def __init__(self, C, D, dtype="f16", T=4, group="cyclic"):
        self.C, self.D, self.T, self.dtype, self.group = C, D, T, dtype, group
        if group == "cyclic":
            self.handle = eqlinear_plan_create(C, D, T, _DTYPE_CODE[dtype])
        else:
            if T % 2:
                raise ValueError("a dihedral group has an even number of elements")
            self.handle = eqlinear_plan_create_group(C, D, GROUPS[group], T // 2,
                                                     _DTYPE_CODE[dtype])

    def close(self):
        if self.handle:
            eqlinear_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass

    def _torch_dtype(self):
        import torch
        return torch.float16 if self.dtype == "f16" else torch.float32

    def _expect(self, t, shape, dtype=None):
        dtype = dtype or self._torch_dtype()
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() \
                or not t.is_cuda:
            raise ValueError(f"expected contiguous CUDA tensor {shape} {dtype}, got "
                             f"{tuple(t.shape)} {t.dtype} contiguous={t.is_contiguous()}")

    def set_weight(self, W, bias=None, stream=None):
        self._expect(W, (self.D, self.C, self.T))
        if bias is not None:
            self._expect(bias, (self.D,))
        eqlinear_set_weight(self.handle, W, bias, stream)

    def forward(self, x, y=None, stream=None, act=None):
        """y = act(layer(x)); act is None, "gelu" or "gelu_tanh" (fused)."""
        import torch
        N = x.shape[0]
        self._expect(x, (N, self.C, self.T))
        if y is None:
            y = torch.empty((N, self.D, self.T), dtype=x.dtype, device=x.device)
        self._expect(y, (N, self.D, self.T))
        if act is None:
            eqlinear_forward(self.handle, x, y, N, stream)
        else:
            eqlinear_forward_act(self.handle, x, y, N, ACTIVATIONS[act], stream)
        return y

    def backward_input(self, dy, dx=None, stream=None):
        import torch
        N = dy.shape[0]
        self._expect(dy, (N, self.D, self.T))
        if dx is None:
            dx = torch.empty((N, self.C, self.T), dtype=dy.dtype, device=dy.device)
        self._expect(dx, (N, self.C, self.T))
        eqlinear_backward_input(self.handle, dy, dx, N, stream)
        return dx

    def workspace_bytes(self, N):
        return eqlinear_backward_weight_workspace(self.handle, N)

    def backward_weight(self, x, dy, dW=None, dbias=None, workspace=None, stream=None,
                        want_bias=True):
        import torch
        N = x.shape[0]
        self._expect(x, (N, self.C, self.T))
        self._expect(dy, (N, self.D, self.T))
        dev = x.device
        if dW is None:
            dW = torch.empty((self.D, self.C, self.T), dtype=torch.float32, device=dev)
        if dbias is None and want_bias:
            dbias = torch.empty((self.D,), dtype=torch.float32, device=dev)
        need = self.workspace_bytes(N)
        if workspace is None:
            workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
        eqlinear_backward_weight(self.handle, x, dy, dW, dbias, N, workspace,
                                 workspace.numel() * workspace.element_size(), stream)
        return dW, dbias

    def mac_counts(self, N):
        return eqlinear_mac_counts(self.handle, N)


class ConvPlan:
    """p4 group convolution plan (k x k kernel, zero padding, stride 1);
    calls take contiguous torch CUDA tensors: f [N, H, W, C, 4],
    y [N, H, W, D, 4], psi [D, C, k, k, 4], bias [D]."""

    def __init__(self, C, D, k=3, dtype="f16"):
        self.C, self.D, self.k, self.dtype = C, D, k, dtype
        self.handle = eqconv_plan_create(C, D, k, _DTYPE_CODE[dtype])

    def close(self):
        if self.handle:
            eqconv_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass

    _torch_dtype = Plan._torch_dtype
    _expect = Plan._expect

    def set_weight(self, psi, bias=None, stream=None):
        self._expect(psi, (self.D, self.C, self.k, self.k, 4))
        if bias is not None:
            self._expect(bias, (self.D,))
        eqconv_set_weight(self.handle, psi, bias, stream)

    def forward(self, f, y=None, stream=None, act=None):
        import torch
        N, H, W = f.shape[:3]
        self._expect(f, (N, H, W, self.C, 4))
        if y is None:
            y = torch.empty((N, H, W, self.D, 4), dtype=f.dtype, device=f.device)
        self._expect(y, (N, H, W, self.D, 4))
        eqconv_forward(self.handle, f, y, N, H, W, ACTIVATIONS[act], stream)
        return y

    def backward_input(self, dy, df=None, stream=None):
        import torch
        N, H, W = dy.shape[:3]
        self._expect(dy, (N, H, W, self.D, 4))
        if df is None:
            df = torch.empty((N, H, W, self.C, 4), dtype=dy.dtype, device=dy.device)
        self._expect(df, (N, H, W, self.C, 4))
        eqconv_backward_input(self.handle, dy, df, N, H, W, stream)
        return df

    def workspace_bytes(self, N, H, W):
        return eqconv_backward_weight_workspace(self.handle, N, H, W)

    def backward_weight(self, f, dy, dpsi=None, dbias=None, workspace=None, stream=None,
                        want_bias=True):
        import torch
        N, H, W = f.shape[:3]
        self._expect(f, (N, H, W, self.C, 4))
        self._expect(dy, (N, H, W, self.D, 4))
        dev = f.device
        if dpsi is None:
            dpsi = torch.empty((self.D, self.C, self.k, self.k, 4), dtype=torch.float32,
                               device=dev)
        if dbias is None and want_bias:
            dbias = torch.empty((self.D,), dtype=torch.float32, device=dev)
        need = self.workspace_bytes(N, H, W)
        if workspace is None:
            workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
        eqconv_backward_weight(self.handle, f, dy, dpsi, dbias, N, H, W, workspace,
                               workspace.numel() * workspace.element_size(), stream)
        return dpsi, dbias

    def mac_counts(self, N, H, W):
        return eqconv_mac_counts(self.handle, N, H, W)
