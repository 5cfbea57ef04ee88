"""Seeded synthetic workloads for the EQ-Linear layer (p4, other cyclic groups,
and p4m) and for the p4 group convolution.

This module holds the workload shapes and the seeded input generators, and
nothing of the layer's arithmetic.  It is the one module shared by the oracle
tests and the HIP path's tests and bench.

The shapes stand in for the linear layers of the equivariant vision models the
Flash EQ-Linear paper accelerates (gist.science summary, "Livello di Rete":
Flash EQ-ViT / Flash EQ-Swin).  The paper's own operator shapes are not given,
so ViT-S-like (64 images x 197 tokens, 384 features) and Swin-like
(64 images x 56 x 56 tokens, 768 features) layers are used, with C and D
counted per group element (a row holds C*T input and D*T output features).
The C8 and p4m workloads keep the ViT-S-like MLP widths (384 -> 1536
features) on a group of order 8 (rotations by 45 degrees; rotations by 90
degrees and reflections), so C and D are half of the p4 ones.

The convolution workloads stand in for an equivariant convolution at the
first stage of a Swin-like network (64 images at 56 x 56, 192 features = 48
channels per rotation, 3 x 3 kernel); the pages name such convolutions as the
next operator and give no shapes ("Limitazioni e Lavoro Futuro").

Drawing rule: numpy PCG64 seeded with ``seed``, draws in the order x, W, bias,
dy, each in fp64, then cast to fp32 and, for fp16 runs, from fp32 to fp16 with
round-to-nearest-even.  The second parameter of every normal distribution is a
variance: x, dy ~ N(0, 1); W ~ N(0, 1/(C*T)) (fan-in scaling); bias ~ N(0, 0.02).
"""
from dataclasses import dataclass
import numpy as np

T_P4 = 4


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    C: int
    D: int
    T: int
    dtypes: tuple
    bias: bool
    passes: tuple  # subset of ("forward", "backward")
    desc: str
    group: str = "cyclic"  # "cyclic" (C_T) or "dihedral" (D_{T/2})


WORKLOADS = {
    "tiny": Workload("tiny", 64, 8, 8, T_P4, ("f32",), False, ("forward",),
                     "tiny p4 layer, 32->32 features"),
    "vit_s_proj": Workload("vit_s_proj", 12608, 96, 96, T_P4, ("f32", "f16"), True, ("forward",),
                           "ViT-S-like projection, 64 images x 197 tokens, 384->384 features"),
    "vit_s_mlp": Workload("vit_s_mlp", 12608, 96, 384, T_P4, ("f16",), True, ("forward",),
                          "ViT-S-like MLP expansion, 64 images x 197 tokens, 384->1536 features"),
    "swin_stage": Workload("swin_stage", 200704, 192, 768, T_P4, ("f16", "f32"), True, ("forward",),
                           "Swin-like stage, 64 images x 56x56 tokens, 768->3072 features"),
    "vit_s_mlp_bwd": Workload("vit_s_mlp_bwd", 12608, 96, 384, T_P4, ("f16",), True, ("backward",),
                              "backward of the ViT-S-like MLP expansion (dX, dW, dbias)"),
    "vit_s_mlp_c8": Workload("vit_s_mlp_c8", 12608, 48, 192, 8, ("f16", "f32"), True,
                             ("forward", "backward"),
                             "ViT-S-like MLP expansion on the rotation group C8, "
                             "64 images x 197 tokens, 384->1536 features"),
    "vit_s_mlp_p4m": Workload("vit_s_mlp_p4m", 12608, 48, 192, 8, ("f16", "f32"), True,
                              ("forward", "backward"),
                              "ViT-S-like MLP expansion on p4m (rotations and reflections, "
                              "the dihedral group D4), 64 images x 197 tokens, "
                              "384->1536 features", group="dihedral"),
}

_NP_DTYPE = {"f32": np.float32, "f16": np.float16}


def _cast(a, dtype):
    a32 = a.astype(np.float32)
    return a32 if dtype == "f32" else a32.astype(np.float16)


def make_inputs(C, D, N, T=T_P4, dtype="f32", seed=0, bias=True, dy=False):
    """Seeded synthetic tensors {x, W, bias, dy} as numpy arrays in ``dtype``.

    x: [N, C, T], W: [D, C, T], bias: [D] or None, dy: [N, D, T] or None.
    """
    if dtype not in _NP_DTYPE:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    out = {}
    out["x"] = _cast(rng.standard_normal((N, C, T)), dtype)
    out["W"] = _cast(rng.standard_normal((D, C, T)) * np.sqrt(1.0 / (C * T)), dtype)
    out["bias"] = _cast(rng.standard_normal(D) * np.sqrt(0.02), dtype) if bias else None
    out["dy"] = _cast(rng.standard_normal((N, D, T)), dtype) if dy else None
    return out


def workload_inputs(name, dtype=None, seed=0):
    w = WORKLOADS[name]
    dt = dtype or w.dtypes[0]
    return make_inputs(w.C, w.D, w.N, w.T, dt, seed, bias=w.bias, dy="backward" in w.passes)


@dataclass(frozen=True)
class ConvWorkload:
    name: str
    N: int
    H: int
    W: int
    C: int
    D: int
    k: int
    dtypes: tuple
    bias: bool
    desc: str


CONV_WORKLOADS = {
    "p4conv_tiny": ConvWorkload("p4conv_tiny", 2, 8, 8, 8, 8, 3, ("f32", "f16"), True,
                                "tiny p4 group convolution, 2 images at 8 x 8, 32->32 features"),
    "p4conv_stage": ConvWorkload("p4conv_stage", 64, 56, 56, 48, 48, 3, ("f16", "f32"), True,
                                 "p4 group convolution 3 x 3 at a Swin-like first stage, "
                                 "64 images at 56 x 56, 192->192 features"),
}


def make_conv_inputs(N, H, W, C, D, k, dtype="f32", seed=0, bias=True, dy=False):
    """Seeded synthetic tensors {f, psi, bias, dy} as numpy arrays in ``dtype``.

    f: [N, H, W, C, 4] ~ N(0, 1); psi: [D, C, k, k, 4] ~ N(0, 1/(4 C k^2))
    (fan-in); bias: [D] ~ N(0, 0.02) or None; dy: [N, H, W, D, 4] ~ N(0, 1) or
    None.  Drawn in that order, as make_inputs."""
    if dtype not in _NP_DTYPE:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    out = {}
    out["f"] = _cast(rng.standard_normal((N, H, W, C, 4)), dtype)
    out["psi"] = _cast(rng.standard_normal((D, C, k, k, 4)) * np.sqrt(1.0 / (4 * C * k * k)), dtype)
    out["bias"] = _cast(rng.standard_normal(D) * np.sqrt(0.02), dtype) if bias else None
    out["dy"] = _cast(rng.standard_normal((N, H, W, D, 4)), dtype) if dy else None
    return out


def conv_workload_inputs(name, dtype=None, seed=0, dy=False):
    w = CONV_WORKLOADS[name]
    dt = dtype or w.dtypes[0]
    return make_conv_inputs(w.N, w.H, w.W, w.C, w.D, w.k, dt, seed, bias=w.bias, dy=dy)


def same_sign_groups(shape, lo, hi, dtype, seed):
    """Seeded tensor of ``shape`` whose group vectors (the last axis) have one
    random sign each and magnitudes uniform in [lo, hi): with lo above
    65504 / T every group sums past the binary16 range while each value stays
    inside it.  For range tests of binary16 paths (loss-scaled gradients and
    large activations)."""
    if dtype not in _NP_DTYPE:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    sign = np.where(rng.random(shape[:-1] + (1,)) < 0.5, -1.0, 1.0)
    mag = lo + (hi - lo) * rng.random(shape)
    return _cast(sign * mag, dtype)
