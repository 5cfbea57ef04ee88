"""Shared helpers of the GPU parity tests: move seeded numpy inputs to the GPU,
run the library through its C ABI, and compare with the oracle."""
import numpy as np

TOL = {"f32": 1e-5, "f16": 2e-3}


def torch_mod():
    import torch
    return torch


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # noqa: BLE001
        return False


def to_dev(a):
    torch = torch_mod()
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def to_np64(t):
    return t.detach().to("cpu").numpy().astype(np.float64)


def rel_err(got, ref):
    """max |got - ref| / max |ref|, in fp64 (the parity metric)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)
