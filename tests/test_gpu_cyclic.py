"""Parity of the cyclic-group path (group sizes 2 <= T <= 16 other than the
p4 kernels' T = 4) with the fp64 oracle, through the C ABI.

Flash EQ-Linear, "Approccio Algoritmico": the same group-DFT method for a
general group size T, keeping the frequencies k <= T/2.  The oracle is the
dense definition for any T, so the bar is the same as for p4:
max|gpu - oracle| / max|oracle| <= 1e-5 (binary32), <= 2e-3 (binary16)."""
import numpy as np
import pytest

import oracle
from group_dft_structured_amd import Plan
from group_dft_structured_amd.workloads import WORKLOADS, make_inputs
from tests.gpu_helpers import TOL, gpu_available, rel_err, to_dev, to_np64, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _sync():
    torch_mod().cuda.synchronize()


def _forward_case(C, D, N, T, dtype, seed=0, bias=True):
    inp = make_inputs(C, D, N, T, dtype=dtype, seed=seed, bias=bias)
    plan = Plan(C, D, dtype, T=T)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    y = plan.forward(to_dev(inp["x"]))
    _sync()
    ref = oracle.forward(inp["x"], inp["W"], inp["bias"])
    err = rel_err(to_np64(y), ref)
    print(f"cyclic forward T={T} C={C} D={D} N={N} {dtype}: rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype], err
    plan.close()


def _backward_case(C, D, N, T, dtype, seed=0):
    inp = make_inputs(C, D, N, T, dtype=dtype, seed=seed, bias=True, dy=True)
    plan = Plan(C, D, dtype, T=T)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
    dx = plan.backward_input(dy)
    dW, db = plan.backward_weight(x, dy)
    _sync()
    ref_dx = oracle.backward_input(inp["dy"], inp["W"])
    ref_dW, ref_db = oracle.backward_weight(inp["x"], inp["dy"])
    e = (rel_err(to_np64(dx), ref_dx), rel_err(to_np64(dW), ref_dW), rel_err(to_np64(db), ref_db))
    print(f"cyclic backward T={T} C={C} D={D} N={N} {dtype}: dx {e[0]:.3e} dW {e[1]:.3e} "
          f"dbias {e[2]:.3e}", flush=True)
    for v in e:
        assert v <= TOL[dtype], e
    plan.close()


GROUPS = [2, 3, 5, 6, 7, 8, 9, 12, 16]


# ragged shapes: channel counts that are not multiples of the 32- or 16-wide
# reduction chunks or the 32/64-wide tiles, row counts with a partial tile
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", GROUPS)
@pytest.mark.parametrize("C,D,N", [(1, 1, 1), (5, 7, 63), (33, 70, 130), (48, 192, 1000)])
def test_cyclic_forward_ragged(C, D, N, T, dtype):
    _forward_case(C, D, N, T, dtype, seed=3 + T)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [2, 3, 8, 11, 16])
@pytest.mark.parametrize("C,D,N", [(5, 7, 63), (33, 70, 600), (70, 33, 700)])
def test_cyclic_backward_ragged(C, D, N, T, dtype):
    _backward_case(C, D, N, T, dtype, seed=5 + T)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_cyclic_path_at_p4(dtype, monkeypatch):
    """T = 4 through the cyclic kernels (a plan created with EQL_CYCLIC_P4=1)."""
    monkeypatch.setenv("EQL_CYCLIC_P4", "1")
    _forward_case(33, 70, 300, 4, dtype, seed=4)
    _backward_case(33, 70, 300, 4, dtype, seed=4)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_cyclic_vit_s_mlp_c8(dtype):
    w = WORKLOADS["vit_s_mlp_c8"]
    _forward_case(w.C, w.D, w.N, w.T, dtype)
    _backward_case(w.C, w.D, w.N, w.T, dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [3, 8])
def test_cyclic_equivariance(T, dtype):
    """Rolling x along the group axis rolls y ("Contributi Chiave": rotation
    equivariance is preserved), for every shift of the group."""
    torch = torch_mod()
    inp = make_inputs(40, 56, 700, T, dtype=dtype, seed=8)
    plan = Plan(40, 56, dtype, T=T)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x = to_dev(inp["x"])
    y = plan.forward(x)
    ymax = float(y.abs().max())
    for r in range(1, T):
        yr = plan.forward(torch.roll(x, r, dims=2).contiguous())
        _sync()
        err = float((yr.float() - torch.roll(y, r, dims=2).float()).abs().max()) / ymax
        assert err <= TOL[dtype], (r, err)
    plan.close()


def test_cyclic_zero_rows_and_determinism():
    torch = torch_mod()
    C, D, T = 48, 192, 8
    inp = make_inputs(C, D, 3000, T, dtype="f16", seed=9, dy=True)
    plan = Plan(C, D, "f16", T=T)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
    # N = 0: forward/backward_input are no-ops, backward_weight writes zeros
    empty_x = torch.empty((0, C, T), dtype=torch.float16, device="cuda")
    empty_dy = torch.empty((0, D, T), dtype=torch.float16, device="cuda")
    assert plan.forward(empty_x).shape == (0, D, T)
    dW0, db0 = plan.backward_weight(empty_x, empty_dy)
    _sync()
    assert float(dW0.abs().max()) == 0.0 and float(db0.abs().max()) == 0.0
    outs = []
    for _ in range(2):
        y = plan.forward(x)
        dx = plan.backward_input(dy)
        dW, db = plan.backward_weight(x, dy)
        _sync()
        outs.append((y.clone(), dx.clone(), dW.clone(), db.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    plan.close()


# every tile shape of the cyclic matrix-core kernel (rows x output channels:
# 0 = 64x64 for T <= 8, 1 = 64x32, 2 = 32x64, 3 = 32x32)
@pytest.mark.parametrize("tile", [0, 1, 2, 3])
@pytest.mark.parametrize("T,dtype", [(3, "f32"), (8, "f16"), (8, "f32"), (12, "f16")])
def test_cyclic_tiles(tile, T, dtype, monkeypatch):
    monkeypatch.setenv("EQL_CYC_TILE", str(tile))
    _forward_case(33, 70, 517, T, dtype, seed=11)
    inp = make_inputs(33, 70, 517, T, dtype=dtype, seed=12, bias=True, dy=True)
    plan = Plan(33, 70, dtype, T=T)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    dx = plan.backward_input(to_dev(inp["dy"]))
    _sync()
    err = rel_err(to_np64(dx), oracle.backward_input(inp["dy"], inp["W"]))
    assert err <= TOL[dtype], err
    plan.close()


# backward_weight tile edges (64 only for T <= 8) and work-group targets,
# which set the number of row splits
@pytest.mark.parametrize("bw_tile,bw_wgs", [(32, 512), (64, 512), (32, 64), (32, 2048)])
@pytest.mark.parametrize("T,dtype", [(3, "f32"), (8, "f16"), (12, "f32")])
def test_cyclic_backward_weight_configs(bw_tile, bw_wgs, T, dtype, monkeypatch):
    monkeypatch.setenv("EQL_CYC_BW_TILE", str(bw_tile))
    monkeypatch.setenv("EQL_CYC_BW_WGS", str(bw_wgs))
    _backward_case(70, 45, 1500, T, dtype, seed=13)


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh"])
@pytest.mark.parametrize("T,dtype", [(3, "f32"), (8, "f16"), (8, "f32"), (16, "f16")])
def test_cyclic_forward_act(T, dtype, act):
    inp = make_inputs(33, 70, 517, T, dtype=dtype, seed=17)
    plan = Plan(33, 70, dtype, T=T)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    y = plan.forward(to_dev(inp["x"]), act=act)
    _sync()
    err = rel_err(to_np64(y), oracle.forward_act(inp["x"], inp["W"], inp["bias"], act))
    assert err <= TOL[dtype], err
    plan.close()
