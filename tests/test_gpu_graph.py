"""The layer's calls (and the group convolution's) captured in a HIP graph and replayed.

Every call is stream-ordered, allocates nothing after the plan's first
set_weight and records no memset, so it can be captured.  Each case captures
forward (plain and with the fused GELU), backward_input and backward_weight
on a side stream, replays the graph several times with eager work of the
program in between (a weight update, an eager forward on other data,
synchronisations), and checks every replay against the eager results, bit for
bit, and the eager results against the oracle."""
import numpy as np
import pytest

import oracle
from group_dft_structured_amd import Plan
from group_dft_structured_amd.workloads import make_inputs
from tests.gpu_helpers import TOL, gpu_available, rel_err, to_dev, to_np64, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


CASES = [
    # (C, D, N, T, group, dtype): p4 on its tuned kernels, p4 binary32, a
    # cyclic group, p4m on paired channels and p4m on the generic kernels
    (96, 384, 3001, 4, "cyclic", "f16"),
    (96, 96, 1000, 4, "cyclic", "f32"),
    (48, 192, 1000, 8, "cyclic", "f16"),
    (48, 192, 1000, 8, "dihedral", "f16"),
    (40, 56, 700, 8, "dihedral", "f32"),
]


@pytest.mark.parametrize("C,D,N,T,group,dtype", CASES)
def test_graph_replays_match_eager(C, D, N, T, group, dtype):
    torch = torch_mod()
    inp = make_inputs(C, D, N, T, dtype=dtype, seed=51, bias=True, dy=True)
    plan = Plan(C, D, dtype, T=T, group=group)
    W, b = to_dev(inp["W"]), to_dev(inp["bias"])
    plan.set_weight(W, b)
    x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
    tdt = x.dtype
    y = torch.empty((N, D, T), dtype=tdt, device="cuda")
    yg = torch.empty_like(y)
    dx = torch.empty((N, C, T), dtype=tdt, device="cuda")
    dW = torch.empty((D, C, T), dtype=torch.float32, device="cuda")
    db = torch.empty((D,), dtype=torch.float32, device="cuda")
    ws = torch.empty((max(plan.workspace_bytes(N), 16),), dtype=torch.uint8, device="cuda")

    def step(stream):
        plan.forward(x, y, stream=stream)
        plan.forward(x, yg, stream=stream, act="gelu")
        plan.backward_input(dy, dx, stream=stream)
        plan.backward_weight(x, dy, dW, db, ws, stream=stream)

    # eager reference
    step(None)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y, yg, dx, dW, db)]
    refs = [oracle.forward(inp["x"], inp["W"], inp["bias"], group=group),
            oracle.forward_act(inp["x"], inp["W"], inp["bias"], "gelu", group=group),
            oracle.backward_input(inp["dy"], inp["W"], group=group),
            *oracle.backward_weight(inp["x"], inp["dy"], group=group)]
    for name, got, ref in zip(("y", "gelu", "dx", "dW", "dbias"), eager, refs):
        err = rel_err(to_np64(got), ref)
        assert err <= TOL[dtype], (name, err)

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(s)  # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            step(s)
    other = torch.randn_like(x.float()).to(tdt)
    W2 = (W.float() * -0.5).to(tdt)
    for rep in range(4):
        for t in (y, yg, dx, dW, db):
            t.fill_(7)
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("y", "gelu", "dx", "dW", "dbias"), (y, yg, dx, dW, db), eager):
            assert torch.equal(got, ref), (rep, name)
        # eager work of the program between replays, on other buffers; the
        # weight changes and is restored, so the captured spectra are reread
        plan.forward(other, torch.empty_like(y))
        plan.set_weight(W2, b)
        plan.forward(other)
        plan.set_weight(W, b)
        torch.cuda.synchronize()
    plan.close()


CONV_CASES = [
    # (N, H, W, C, D, k, dtype): the register-direct binary16 kernel, the
    # LDS-tiled binary32 one
    (2, 12, 10, 48, 48, 3, "f16"),
    (1, 9, 11, 8, 12, 3, "f32"),
]


@pytest.mark.parametrize("N,H,W,C,D,k,dtype", CONV_CASES)
def test_conv_graph_replays_match_eager(N, H, W, C, D, k, dtype):
    """The convolution's calls captured in a graph and replayed between
    eager work, bit-identical to eager and within the oracle bar."""
    from group_dft_structured_amd import ConvPlan
    from group_dft_structured_amd.workloads import make_conv_inputs
    torch = torch_mod()
    inp = make_conv_inputs(N, H, W, C, D, k, dtype=dtype, seed=52, bias=True, dy=True)
    plan = ConvPlan(C, D, k, dtype)
    psi, b = to_dev(inp["psi"]), to_dev(inp["bias"])
    plan.set_weight(psi, b)
    f, dy = to_dev(inp["f"]), to_dev(inp["dy"])
    y = torch.empty((N, H, W, D, 4), dtype=f.dtype, device="cuda")
    yg = torch.empty_like(y)
    df = torch.empty_like(f)
    dpsi = torch.empty((D, C, k, k, 4), dtype=torch.float32, device="cuda")
    db = torch.empty((D,), dtype=torch.float32, device="cuda")
    ws = torch.empty((plan.workspace_bytes(N, H, W),), dtype=torch.uint8, device="cuda")

    def step(stream):
        plan.forward(f, y, stream=stream)
        plan.forward(f, yg, stream=stream, act="gelu")
        plan.backward_input(dy, df, stream=stream)
        plan.backward_weight(f, dy, dpsi, db, ws, stream=stream)

    step(None)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y, yg, df, dpsi, db)]
    refs = [oracle.conv_forward(inp["f"], inp["psi"], inp["bias"]),
            oracle.conv_forward_act(inp["f"], inp["psi"], inp["bias"], "gelu"),
            oracle.conv_backward_input(inp["dy"], inp["psi"]),
            *oracle.conv_backward_weight(inp["f"], inp["dy"], k)]
    for name, got, ref in zip(("y", "gelu", "df", "dpsi", "dbias"), eager, refs):
        assert rel_err(to_np64(got), ref) <= TOL[dtype], name

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(s)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            step(s)
    other = torch.randn_like(f.float()).to(f.dtype)
    psi2 = (psi.float() * 0.5).to(psi.dtype)
    for rep in range(4):
        for t in (y, yg, df, dpsi, db):
            t.fill_(7)
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("y", "gelu", "df", "dpsi", "dbias"), (y, yg, df, dpsi, db), eager):
            assert torch.equal(got, ref), (rep, name)
        plan.forward(other, torch.empty_like(y))
        plan.set_weight(psi2, b)
        plan.forward(other)
        plan.set_weight(psi, b)
        torch.cuda.synchronize()
    plan.close()
