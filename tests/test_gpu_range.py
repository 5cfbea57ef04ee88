"""Binary16 input range of every binary16 path, against the fp64 oracle.

The inputs are group vectors whose four (or T) values share one sign and lie
in the upper half of the binary16 range, so every group sum exceeds 65504
while each value and each output stays inside the range.  A dense layer with
binary16 inputs and fp32 accumulation computes these exactly up to rounding;
so must the spectral path, whose planes carry a power-of-two scaling that
bounds them by the largest input magnitude.  Weights are the usual fan-in
draws divided by 8 (exact), which keeps the outputs inside the binary16
range.  Bar: max|gpu - oracle| / max|oracle| <= 2e-3 per output tensor."""
import numpy as np
import pytest

import oracle
from group_dft_structured_amd import ConvPlan, Plan
from group_dft_structured_amd.workloads import make_conv_inputs, make_inputs, same_sign_groups
from tests.gpu_helpers import TOL, gpu_available, rel_err, to_dev, to_np64, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _sync():
    torch_mod().cuda.synchronize()


def _large(shape, T, seed):
    """Same-sign groups whose sum is at least 1.05 x 65504."""
    lo = 1.05 * 65504.0 / T
    return same_sign_groups(shape, lo, 1.1 * lo, "f16", seed)


def _small_weight(inp):
    return (inp["W"].astype(np.float32) / 8).astype(np.float16)


def _assert_close(name, got, ref):
    err = rel_err(to_np64(got), ref)
    print(f"{name}: rel err {err:.3e}", flush=True)
    assert np.isfinite(err) and err <= TOL["f16"], (name, err)


P4_FWD = {
    "ws_default": {},
    "ws_split": {"EQL_WS_SMALL_MB": "0"},
    "ws_stream": {"EQL_WS_OUT": "1"},
    "tiled": {"EQL_NO_WS": "1"},
}


@pytest.mark.parametrize("act", [None, "gelu"])
@pytest.mark.parametrize("path", sorted(P4_FWD))
def test_p4_forward_large_groups(path, act, monkeypatch):
    for k, v in P4_FWD[path].items():
        monkeypatch.setenv(k, v)
    C, D, N = 96, 384, 3001
    inp = make_inputs(C, D, N, dtype="f16", seed=41)
    W = _small_weight(inp)
    x = _large((N, C, 4), 4, seed=42)
    plan = Plan(C, D, "f16")
    plan.set_weight(to_dev(W), to_dev(inp["bias"]))
    y = plan.forward(to_dev(x), act=act)
    _sync()
    ref = oracle.forward_act(x, W, inp["bias"], act) if act else oracle.forward(x, W, inp["bias"])
    _assert_close(f"p4 forward {path} act={act}", y, ref)
    plan.close()


@pytest.mark.parametrize("path", ["ws", "tiled"])
def test_p4_backward_input_large_groups(path, monkeypatch):
    if path == "tiled":
        monkeypatch.setenv("EQL_NO_WS", "1")
    C, D, N = 96, 384, 3001
    inp = make_inputs(C, D, N, dtype="f16", seed=43)
    W = _small_weight(inp)
    dy = _large((N, D, 4), 4, seed=44)
    plan = Plan(C, D, "f16")
    plan.set_weight(to_dev(W), None)
    dx = plan.backward_input(to_dev(dy))
    _sync()
    _assert_close(f"p4 backward_input {path}", dx, oracle.backward_input(dy, W))
    plan.close()


@pytest.mark.parametrize("path", ["ws", "tiled"])
def test_p4_backward_weight_large_groups(path, monkeypatch):
    if path == "tiled":
        monkeypatch.setenv("EQL_BW_TILED", "1")
    C, D, N = 96, 384, 3001
    inp = make_inputs(C, D, N, dtype="f16", seed=45)
    x = _large((N, C, 4), 4, seed=46)
    dy = _large((N, D, 4), 4, seed=47)
    plan = Plan(C, D, "f16")
    plan.set_weight(to_dev(_small_weight(inp)), None)
    dW, db = plan.backward_weight(to_dev(x), to_dev(dy))
    _sync()
    ref_dW, ref_db = oracle.backward_weight(x, dy)
    _assert_close(f"p4 dW {path}", dW, ref_dW)
    _assert_close(f"p4 dbias {path}", db, ref_db)
    plan.close()


# the generic group kernels: cyclic groups (plane scaling 1/4 for T = 3,
# 1/8 for T = 8) and p4m on the paired p4 kernels and on the group Fourier
# transform
GROUP_CASES = [
    ("cyclic", 3, {}),
    ("cyclic", 8, {}),
    ("dihedral", 8, {}),
    ("dihedral", 8, {"EQL_P4M_PAIRS": "0"}),
    ("dihedral", 6, {}),
]


@pytest.mark.parametrize("group,T,env", GROUP_CASES, ids=lambda v: str(v))
def test_group_large_groups(group, T, env, monkeypatch):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    C, D, N = 48, 192, 1001
    inp = make_inputs(C, D, N, T, dtype="f16", seed=48)
    W = _small_weight(inp)
    x = _large((N, C, T), T, seed=49)
    dy = _large((N, D, T), T, seed=50)
    plan = Plan(C, D, "f16", T=T, group=group)
    plan.set_weight(to_dev(W), to_dev(inp["bias"]))
    y = plan.forward(to_dev(x))
    dx = plan.backward_input(to_dev(dy))
    dW, db = plan.backward_weight(to_dev(x), to_dev(dy))
    _sync()
    tag = f"{group} T={T} {env}"
    _assert_close(f"{tag} forward", y, oracle.forward(x, W, inp["bias"], group=group))
    _assert_close(f"{tag} backward_input", dx, oracle.backward_input(dy, W, group=group))
    ref_dW, ref_db = oracle.backward_weight(x, dy, group=group)
    _assert_close(f"{tag} dW", dW, ref_dW)
    _assert_close(f"{tag} dbias", db, ref_db)
    plan.close()


def test_conv_large_groups():
    """The group convolution: register-direct forward and backward input,
    filter gradient through the patch layer's weight gradient."""
    N, H, W_, C, D, k = 2, 9, 10, 48, 48, 3
    inp = make_conv_inputs(N, H, W_, C, D, k, dtype="f16", seed=51)
    psi = (inp["psi"].astype(np.float32) / 8).astype(np.float16)
    f = _large((N, H, W_, C, 4), 4, seed=52)
    dy = _large((N, H, W_, D, 4), 4, seed=53)
    plan = ConvPlan(C, D, k, "f16")
    plan.set_weight(to_dev(psi), to_dev(inp["bias"]))
    y = plan.forward(to_dev(f))
    df = plan.backward_input(to_dev(dy))
    dpsi, dbias = plan.backward_weight(to_dev(f), to_dev(dy))
    _sync()
    _assert_close("conv forward", y, oracle.conv_forward(f, psi, inp["bias"]))
    _assert_close("conv backward_input", df, oracle.conv_backward_input(dy, psi))
    rpsi, rbias = oracle.conv_backward_weight(f, dy, k)
    _assert_close("conv dpsi", dpsi, rpsi)
    _assert_close("conv dbias", dbias, rbias)
    plan.close()
