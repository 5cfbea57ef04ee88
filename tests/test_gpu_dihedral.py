"""Parity of the dihedral-group path (D_n, 2 <= n <= 8, p4m = D_4) with the
fp64 oracle, through the C ABI.

Reading: the reflection groups that "Limitazioni e Lavoro Futuro" names as
the next groups, with the layer as the group convolution
y[g] = sum_h W[h^-1 g] x[h] (the circular convolution for the cyclic group).
The oracle is the dense group matrix of that definition, so the bar is the
same as for p4: max|gpu - oracle| / max|oracle| <= 1e-5 (binary32),
<= 2e-3 (binary16)."""
import numpy as np
import pytest

import oracle
from group_dft_structured_amd import Plan
from group_dft_structured_amd.workloads import WORKLOADS, make_inputs
from tests.gpu_helpers import TOL, gpu_available, rel_err, to_dev, to_np64, torch_mod

pytestmark = pytest.mark.gpu
DIH = "dihedral"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _sync():
    torch_mod().cuda.synchronize()


def _forward_case(C, D, N, n, dtype, seed=0, bias=True, act=None):
    T = 2 * n
    inp = make_inputs(C, D, N, T, dtype=dtype, seed=seed, bias=bias)
    plan = Plan(C, D, dtype, T=T, group=DIH)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    y = plan.forward(to_dev(inp["x"]), act=act)
    _sync()
    ref = oracle.forward_act(inp["x"], inp["W"], inp["bias"], act, group=DIH)
    err = rel_err(to_np64(y), ref)
    print(f"dihedral forward n={n} C={C} D={D} N={N} {dtype} act={act}: rel err {err:.3e}",
          flush=True)
    assert err <= TOL[dtype], err
    plan.close()


def _backward_case(C, D, N, n, dtype, seed=0):
    T = 2 * n
    inp = make_inputs(C, D, N, T, dtype=dtype, seed=seed, bias=True, dy=True)
    plan = Plan(C, D, dtype, T=T, group=DIH)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
    dx = plan.backward_input(dy)
    dW, db = plan.backward_weight(x, dy)
    _sync()
    ref_dx = oracle.backward_input(inp["dy"], inp["W"], group=DIH)
    ref_dW, ref_db = oracle.backward_weight(inp["x"], inp["dy"], group=DIH)
    e = (rel_err(to_np64(dx), ref_dx), rel_err(to_np64(dW), ref_dW), rel_err(to_np64(db), ref_db))
    print(f"dihedral backward n={n} C={C} D={D} N={N} {dtype}: dx {e[0]:.3e} dW {e[1]:.3e} "
          f"dbias {e[2]:.3e}", flush=True)
    for v in e:
        assert v <= TOL[dtype], e
    plan.close()


# ragged shapes: channel counts that are not multiples of the reduction
# chunks or the tiles, row counts with a partial tile
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("C,D,N", [(1, 1, 1), (5, 7, 63), (33, 70, 130), (48, 192, 1000)])
def test_dihedral_forward_ragged(C, D, N, n, dtype):
    _forward_case(C, D, N, n, dtype, seed=21 + n)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n", [2, 3, 4, 7, 8])
@pytest.mark.parametrize("C,D,N", [(5, 7, 63), (33, 70, 600), (70, 33, 700)])
def test_dihedral_backward_ragged(C, D, N, n, dtype):
    _backward_case(C, D, N, n, dtype, seed=23 + n)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_p4m_vit_s_mlp(dtype):
    w = WORKLOADS["vit_s_mlp_p4m"]
    assert w.group == DIH and w.T == 8
    _forward_case(w.C, w.D, w.N, w.T // 2, dtype)
    _backward_case(w.C, w.D, w.N, w.T // 2, dtype)


def _left_perm(n):
    """perm_a[h] = index of a^-1 h in D_n for every a, from the 2 x 2
    orthogonal representation (rotation by 2 pi / n, reflection diag(1, -1))."""
    def mat(u):
        m, r = divmod(u, n)
        c, s = np.cos(2 * np.pi * r / n), np.sin(2 * np.pi * r / n)
        M = np.array([[c, -s], [s, c]])
        return M @ np.diag([1.0, -1.0]) if m else M
    mats = [mat(u) for u in range(2 * n)]
    look = lambda M: int(np.argmin([np.abs(M - Q).max() for Q in mats]))
    return [[look(mats[a].T @ mats[h]) for h in range(2 * n)] for a in range(2 * n)]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n", [3, 4])
def test_dihedral_equivariance(n, dtype):
    """Rotating or reflecting x along the group axis (left translation by any
    element a: x -> x[a^-1 h]) transforms y the same way."""
    torch = torch_mod()
    T = 2 * n
    inp = make_inputs(40, 56, 700, T, dtype=dtype, seed=28)
    plan = Plan(40, 56, dtype, T=T, group=DIH)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x = to_dev(inp["x"])
    y = plan.forward(x)
    ymax = float(y.abs().max())
    for a, perm in enumerate(_left_perm(n)):
        idx = torch.tensor(perm, device="cuda")
        ya = plan.forward(x.index_select(2, idx).contiguous())
        _sync()
        err = float((ya.float() - y.index_select(2, idx).float()).abs().max()) / ymax
        assert err <= TOL[dtype], (a, err)
    plan.close()


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh"])
@pytest.mark.parametrize("n,dtype", [(3, "f32"), (4, "f16"), (4, "f32"), (8, "f16")])
def test_dihedral_forward_act(n, dtype, act):
    _forward_case(33, 70, 517, n, dtype, seed=27, act=act)


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
@pytest.mark.parametrize("n,dtype", [(4, "f16"), (4, "f32"), (6, "f16")])
def test_dihedral_tiles(tile, n, dtype, monkeypatch):
    """Every tile shape of the generic matrix-core kernel (rows x output
    channels: 0 = 64x64 for T <= 8, 1 = 64x32, 2 = 32x64, 3 = 32x32)."""
    monkeypatch.setenv("EQL_CYC_TILE", str(tile))
    _forward_case(33, 70, 517, n, dtype, seed=29)
    _backward_case(33, 70, 517, n, dtype, seed=30)


def test_dihedral_zero_rows_and_determinism():
    torch = torch_mod()
    C, D, T = 48, 192, 8
    inp = make_inputs(C, D, 3000, T, dtype="f16", seed=31, dy=True)
    plan = Plan(C, D, "f16", T=T, group=DIH)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
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


# p4m in binary16 at widths the p4 producer/consumer kernels take runs as the
# p4 layer on paired channels (2C -> 2D); the same shapes with
# EQL_P4M_PAIRS=0 run the group Fourier transform.  Both against the oracle,
# and against each other.
@pytest.mark.parametrize("C,D,N", [(16, 32, 517), (48, 192, 1000), (96, 64, 301), (48, 192, 12608)])
def test_p4m_paired_path(C, D, N, monkeypatch):
    torch = torch_mod()
    inp = make_inputs(C, D, N, 8, dtype="f16", seed=41, bias=True, dy=True)
    outs = {}
    for pairs in ("1", "0"):
        monkeypatch.setenv("EQL_P4M_PAIRS", pairs)
        plan = Plan(C, D, "f16", T=8, group=DIH)
        assert plan.mac_counts(1)[0] == (24 if pairs == "1" else 12) * C * D
        plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
        x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
        y = plan.forward(x)
        yg = plan.forward(x, act="gelu")
        dx = plan.backward_input(dy)
        dW, db = plan.backward_weight(x, dy)
        dW2, _ = plan.backward_weight(x, dy, want_bias=False)
        _sync()
        outs[pairs] = [to_np64(t) for t in (y, yg, dx, dW, db)]
        assert torch.equal(dW, dW2)
        plan.close()
    refs = [oracle.forward(inp["x"], inp["W"], inp["bias"], group=DIH),
            oracle.forward_act(inp["x"], inp["W"], inp["bias"], "gelu", group=DIH),
            oracle.backward_input(inp["dy"], inp["W"], group=DIH),
            *oracle.backward_weight(inp["x"], inp["dy"], group=DIH)]
    for name, a, b, ref in zip(("y", "gelu", "dx", "dW", "dbias"), outs["1"], outs["0"], refs):
        ea, eb = rel_err(a, ref), rel_err(b, ref)
        print(f"p4m paired C={C} D={D} N={N} {name}: paired {ea:.2e} generic {eb:.2e}", flush=True)
        assert ea <= TOL["f16"] and eb <= TOL["f16"], (name, ea, eb)
