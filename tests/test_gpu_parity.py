"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bar: max|gpu - oracle| / max|oracle| <= 1e-5 for binary32 and <= 2e-3 for
binary16 (fp32 accumulation), per output tensor.  The oracle consumes the
exact dtype-rounded inputs widened to fp64."""
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


def run_forward(C, D, N, dtype, seed=0, bias=True):
    inp = make_inputs(C, D, N, dtype=dtype, seed=seed, bias=bias)
    plan = Plan(C, D, dtype)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    y = plan.forward(to_dev(inp["x"]))
    _sync()
    return inp, plan, y


def check_forward_full(C, D, N, dtype, seed=0, bias=True):
    inp, plan, y = run_forward(C, D, N, dtype, seed, bias)
    ref = oracle.forward(inp["x"], inp["W"], inp["bias"])
    err = rel_err(to_np64(y), ref)
    print(f"forward C={C} D={D} N={N} {dtype} bias={bias}: rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype], err
    return err


# ---- workloads at full size ------------------------------------------------

def test_forward_tiny_f32():
    w = WORKLOADS["tiny"]
    check_forward_full(w.C, w.D, w.N, "f32", bias=False)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_forward_vit_s_proj(dtype):
    w = WORKLOADS["vit_s_proj"]
    check_forward_full(w.C, w.D, w.N, dtype)


def test_forward_vit_s_mlp_f16():
    w = WORKLOADS["vit_s_mlp"]
    check_forward_full(w.C, w.D, w.N, "f16")


def _compare_in_blocks(y, ref_fn, x_rows, block=8192):
    """max |y - ref| / max |ref| over the whole tensor, with the oracle and the
    device-to-host copy taken in row blocks (the fp64 oracle output of the
    full Swin-like stage would be 4.9 GB)."""
    err_max = ref_max = 0.0
    for r0 in range(0, x_rows, block):
        r1 = min(x_rows, r0 + block)
        ref = ref_fn(r0, r1)
        got = to_np64(y[r0:r1])
        err_max = max(err_max, float(np.abs(got - ref).max()))
        ref_max = max(ref_max, float(np.abs(ref).max()))
    return err_max / ref_max


@pytest.mark.parametrize("dtype,act", [("f16", None), ("f32", None), ("f16", "gelu")])
def test_forward_swin_stage_full(dtype, act):
    """Full-size Swin-like stage in the launch configuration the benchmark
    times (outputs beyond the memory-side cache: split producer/consumer
    stores), every row against the oracle."""
    w = WORKLOADS["swin_stage"]
    inp = make_inputs(w.C, w.D, w.N, dtype=dtype, seed=0, bias=True)
    plan = Plan(w.C, w.D, dtype)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    y = plan.forward(to_dev(inp["x"]), act=act)
    _sync()
    x, W, b = inp["x"], inp["W"], inp["bias"]
    if act is None:
        ref_fn = lambda r0, r1: oracle.forward(x[r0:r1], W, b)  # noqa: E731
    else:
        ref_fn = lambda r0, r1: oracle.forward_act(x[r0:r1], W, b, act)  # noqa: E731
    err = _compare_in_blocks(y, ref_fn, w.N)
    print(f"swin_stage {dtype} act={act} full: rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype], err
    plan.close()


def _backward_case(C, D, N, dtype, seed=0):
    inp = make_inputs(C, D, N, dtype=dtype, seed=seed, bias=True, dy=True)
    plan = Plan(C, D, dtype)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
    dx = plan.backward_input(dy)
    dW, db = plan.backward_weight(x, dy)
    _sync()
    ref_dx = oracle.backward_input(inp["dy"], inp["W"])
    ref_dW, ref_db = oracle.backward_weight(inp["x"], inp["dy"])
    e = (rel_err(to_np64(dx), ref_dx), rel_err(to_np64(dW), ref_dW), rel_err(to_np64(db), ref_db))
    print(f"backward C={C} D={D} N={N} {dtype}: dx {e[0]:.3e} dW {e[1]:.3e} dbias {e[2]:.3e}",
          flush=True)
    for v in e:
        assert v <= TOL[dtype], e
    return plan, x, dy, dx, dW, db


def test_backward_vit_s_mlp_f16():
    w = WORKLOADS["vit_s_mlp_bwd"]
    _backward_case(w.C, w.D, w.N, "f16")


def test_backward_f32_small():
    _backward_case(96, 384, 3000, "f32")


# ---- ragged shapes and edge cases -------------------------------------------

@pytest.mark.parametrize("kernel", ["auto", "tiled"])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("C,D,N", [(8, 8, 1), (5, 7, 63), (33, 130, 65), (96, 96, 1000),
                                   (1, 1, 129), (64, 256, 257), (130, 33, 70), (200, 72, 191),
                                   (96, 384, 3001), (192, 200, 777), (40, 48, 17)])
def test_forward_ragged(C, D, N, dtype, kernel, monkeypatch):
    """kernel=auto lets the library pick; kernel=tiled forces the general
    tiled kernel for every shape."""
    if kernel == "tiled":
        for k in ("EQL_NO_WS", "EQL_NO_WS32"):
            monkeypatch.setenv(k, "1")
    check_forward_full(C, D, N, dtype, seed=C * 1000 + D)


# binary16 forward paths forced one at a time (each falls back to the general
# tiled kernel where a shape is outside its limits).  EQL_WS_SMALL_MB=0 makes
# every output count as beyond the memory-side cache, so the split
# producer/consumer stores of the largest layers run on ragged shapes.
F16_PATHS = {
    "ws_stream": {"EQL_WS_OUT": "1"},
    "ws_default": {},
    "ws_split": {"EQL_WS_SMALL_MB": "0"},
    "ws_large_unsplit": {"EQL_WS_SMALL_MB": "0", "EQL_WS_SPLIT": "0"},
    "ws_8x1": {"EQL_WS_NC": "8", "EQL_WS_NB": "1"},
    "tiled": {"EQL_NO_WS": "1"},
}


@pytest.mark.parametrize("path", sorted(F16_PATHS))
@pytest.mark.parametrize("C,D,N", [(8, 8, 1), (32, 4, 17), (64, 256, 257), (96, 96, 1000),
                                   (96, 384, 3001), (128, 132, 4001), (160, 36, 255),
                                   (192, 200, 777), (192, 768, 1531)])
def test_forward_f16_paths(C, D, N, path, monkeypatch):
    for k, v in F16_PATHS[path].items():
        monkeypatch.setenv(k, v)
    check_forward_full(C, D, N, "f16", seed=C * 1000 + D + 7)


# every compiled (consumer waves, producer waves, 16-channel blocks per
# consumer, 32-channel reduction steps) case of the producer/consumer kernel
WS_CASES = [(4, 4, 2, 1), (4, 4, 2, 2), (4, 4, 2, 3), (8, 4, 1, 1), (8, 4, 1, 2), (8, 4, 1, 3),
            (8, 4, 1, 4), (8, 4, 1, 5), (8, 4, 1, 6), (4, 4, 1, 8), (4, 4, 1, 12), (3, 4, 1, 8),
            (3, 4, 1, 12)]


@pytest.mark.parametrize("nc,np_,nb,ks", WS_CASES)
def test_forward_ws_cases(nc, np_, nb, ks, monkeypatch):
    """Each case with its output store paths (producer stores written through
    the L2, consumer stores streamed, and the split and unsplit producer
    stores of outputs beyond the memory-side cache) and both producer unit
    shapes (output width 264 is not a multiple of any channel range, so the
    last range is ragged)."""
    monkeypatch.setenv("EQL_WS_NC", str(nc))
    monkeypatch.setenv("EQL_WS_NP", str(np_))
    monkeypatch.setenv("EQL_WS_NB", str(nb))
    for out, g8, small, split in (("0", "0", None, None), ("1", "1", None, None),
                                  ("0", "1", "0", "1"), ("0", "0", "0", "0")):
        monkeypatch.setenv("EQL_WS_OUT", out)
        monkeypatch.setenv("EQL_WS_G8", g8)
        for k, v in (("EQL_WS_SMALL_MB", small), ("EQL_WS_SPLIT", split)):
            if v is None:
                monkeypatch.delenv(k, raising=False)
            else:
                monkeypatch.setenv(k, v)
        check_forward_full(32 * ks, 264, 1234 + ks, "f16", seed=nc * 100 + ks)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("C,D,N", [(8, 8, 1), (5, 7, 63), (33, 130, 600), (130, 33, 1100),
                                   (96, 96, 513)])
def test_backward_ragged(C, D, N, dtype):
    _backward_case(C, D, N, dtype, seed=7 + C)


# every compiled (consumer waves, producer waves, 16-channel reduction
# blocks) case of the binary32 producer/consumer forward, both store policies
WS32_CASES = [(6, 2, 6), (4, 2, 6), (6, 2, 2), (6, 2, 4), (8, 2, 2), (8, 2, 4), (4, 4, 8), (4, 4, 12)]


@pytest.mark.parametrize("nc,np_,kb", WS32_CASES)
def test_forward_ws32_cases(nc, np_, kb, monkeypatch):
    monkeypatch.setenv("EQL_WS32_NC", str(nc))
    monkeypatch.setenv("EQL_WS32_NP", str(np_))
    for stream in ("0", "1"):
        monkeypatch.setenv("EQL_WS32_STREAM", stream)
        check_forward_full(16 * kb, 264, 1234 + kb, "f32", seed=nc * 100 + kb)


F32_PATHS = {"ws32": {}, "tiled": {"EQL_NO_WS32": "1"},
             # one consumer wave per output block over the whole reduction
             "ws32_whole": {"EQL_WS32_NC": "6"},
             # two consumer waves per output block over the reduction halves;
             # the last round of tiles cut into (tile, output block) units
             # where they fit one per worker, or run as whole tiles
             "ws32_split": {"EQL_WS32_NC": "12"},
             "ws32_split_whole_tiles": {"EQL_WS32_NC": "12", "EQL_WS32_TAIL": "0"}}


@pytest.mark.parametrize("path", sorted(F32_PATHS))
@pytest.mark.parametrize("C,D,N", [(16, 4, 3), (96, 96, 12608), (48, 100, 999), (192, 768, 2049),
                                   (64, 36, 257), (96, 40, 1001), (96, 96, 17), (96, 96, 4097)])
def test_forward_f32_paths(C, D, N, path, monkeypatch):
    for k, v in F32_PATHS[path].items():
        monkeypatch.setenv(k, v)
    check_forward_full(C, D, N, "f32", seed=C * 1000 + D + 11)


# backward-input paths forced one at a time (binary16)
BI_PATHS = {
    "ws": {},
    "ws_no_ksplit": {"EQL_WS_KSPLIT": "0"},
    "tiled": {"EQL_NO_WS": "1"},
}


@pytest.mark.parametrize("path", sorted(BI_PATHS))
@pytest.mark.parametrize("C,D,N", [(96, 384, 12608), (96, 384, 1001), (32, 256, 333), (100, 96, 777),
                                   (64, 288, 65), (96, 384, 2063), (48, 384, 17), (144, 384, 700),
                                   (100, 384, 300)])
def test_backward_input_paths(C, D, N, path, monkeypatch):
    for k, v in BI_PATHS[path].items():
        monkeypatch.setenv(k, v)
    inp = make_inputs(C, D, N, dtype="f16", seed=C * 7 + D + N, bias=True, dy=True)
    plan = Plan(C, D, "f16")
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    dx = plan.backward_input(to_dev(inp["dy"]))
    _sync()
    err = rel_err(to_np64(dx), oracle.backward_input(inp["dy"], inp["W"]))
    print(f"backward_input {path} C={C} D={D} N={N}: rel err {err:.3e}", flush=True)
    assert err <= TOL["f16"], err


# backward-weight paths forced one at a time (binary16)
BW_PATHS = {
    "ws": {},
    "ws_few_splits": {"EQL_BWS_S": "3"},
    "tiled": {"EQL_BW_TILED": "1"},
}


@pytest.mark.parametrize("path", sorted(BW_PATHS))
@pytest.mark.parametrize("C,D,N", [(2, 2, 1), (32, 34, 95), (96, 384, 3001), (96, 100, 12608),
                                   (64, 256, 777), (192, 66, 530)])
def test_backward_weight_paths(C, D, N, path, monkeypatch):
    for k, v in BW_PATHS[path].items():
        monkeypatch.setenv(k, v)
    inp = make_inputs(C, D, N, dtype="f16", seed=C + D + N, bias=True, dy=True)
    plan = Plan(C, D, "f16")
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    dW, db = plan.backward_weight(to_dev(inp["x"]), to_dev(inp["dy"]))
    _sync()
    ref_dW, ref_db = oracle.backward_weight(inp["x"], inp["dy"])
    e = (rel_err(to_np64(dW), ref_dW), rel_err(to_np64(db), ref_db))
    print(f"backward_weight {path} C={C} D={D} N={N}: dW {e[0]:.3e} dbias {e[1]:.3e}", flush=True)
    assert max(e) <= TOL["f16"], e


def test_backward_weight_calls_in_a_row():
    """Weight-gradient calls of one plan in a row, with split counts that
    change from call to call, each match the
    oracle, and a repeated shape repeats its bits; a plan that never had a
    set_weight gives the same gradient."""
    torch = torch_mod()
    C, D = 96, 384
    bare = Plan(C, D, "f16")
    inp = make_inputs(C, D, 777, dtype="f16", seed=70, bias=True, dy=True)
    dW, db = bare.backward_weight(to_dev(inp["x"]), to_dev(inp["dy"]))
    _sync()
    ref_dW, ref_db = oracle.backward_weight(inp["x"], inp["dy"])
    assert max(rel_err(to_np64(dW), ref_dW), rel_err(to_np64(db), ref_db)) <= TOL["f16"]
    bare.close()
    plan = Plan(C, D, "f16")
    w = make_inputs(C, D, 1, dtype="f16", seed=71, bias=True)
    plan.set_weight(to_dev(w["W"]), to_dev(w["bias"]))
    first = None
    for i, N in enumerate((3001, 12608, 95, 1, 3001)):
        inp = make_inputs(C, D, N, dtype="f16", seed=72 if N == 3001 else 73 + i,
                          bias=True, dy=True)
        dW, db = plan.backward_weight(to_dev(inp["x"]), to_dev(inp["dy"]))
        _sync()
        ref_dW, ref_db = oracle.backward_weight(inp["x"], inp["dy"])
        e = (rel_err(to_np64(dW), ref_dW), rel_err(to_np64(db), ref_db))
        print(f"backward_weight call {i} N={N}: dW {e[0]:.3e} dbias {e[1]:.3e}", flush=True)
        assert max(e) <= TOL["f16"], (N, e)
        if N == 3001:
            if first is None:
                first = (dW.clone(), db.clone())
            else:
                assert torch.equal(first[0], dW) and torch.equal(first[1], db)
    plan.close()


def test_no_bias_equals_zero_bias():
    inp = make_inputs(24, 40, 100, dtype="f32", seed=3, bias=True)
    plan = Plan(24, 40, "f32")
    x = to_dev(inp["x"])
    plan.set_weight(to_dev(inp["W"]), None)
    y0 = plan.forward(x).clone()
    plan.set_weight(to_dev(inp["W"]), to_dev(np.zeros(40, np.float32)))
    y1 = plan.forward(x)
    _sync()
    assert torch_mod().equal(y0, y1)


def test_zero_rows_is_noop():
    torch = torch_mod()
    inp = make_inputs(16, 16, 4, dtype="f16", seed=1)
    plan = Plan(16, 16, "f16")
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x = torch.empty((0, 16, 4), dtype=torch.float16, device="cuda")
    y = plan.forward(x)
    dx = plan.backward_input(torch.empty((0, 16, 4), dtype=torch.float16, device="cuda"))
    dW = torch.full((16, 16, 4), 7.0, device="cuda")
    db = torch.full((16,), 7.0, device="cuda")
    plan.backward_weight(x, torch.empty((0, 16, 4), dtype=torch.float16, device="cuda"), dW, db)
    _sync()
    assert y.shape == (0, 16, 4) and dx.shape == (0, 16, 4)
    assert float(dW.abs().max()) == 0.0 and float(db.abs().max()) == 0.0


# ---- invariants on the GPU ---------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_gpu_equivariance(dtype):
    """Rolling x along the group axis rolls y ("Contributi Chiave": rotation
    equivariance is preserved).  The DFT of a rolled quad is a sign/swap of
    the planes, so the GPU result is rolled exactly up to accumulation order."""
    torch = torch_mod()
    inp = make_inputs(96, 96, 2048, dtype=dtype, seed=5)
    plan = Plan(96, 96, dtype)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x = to_dev(inp["x"])
    y = plan.forward(x)
    ymax = float(y.abs().max())
    for r in (1, 2, 3):
        yr = plan.forward(torch.roll(x, r, dims=2).contiguous())
        _sync()
        err = float((yr.float() - torch.roll(y, r, dims=2).float()).abs().max()) / ymax
        assert err <= TOL[dtype], (r, err)


def test_determinism_bitwise():
    torch = torch_mod()
    w = WORKLOADS["vit_s_mlp_bwd"]
    inp = make_inputs(w.C, w.D, w.N, dtype="f16", seed=9, dy=True)
    plan = Plan(w.C, w.D, "f16")
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
    outs = []
    for _ in range(2):
        y = plan.forward(x)
        dx = plan.backward_input(dy)
        dW, db = plan.backward_weight(x, dy)
        _sync()
        outs.append((y.clone(), dx.clone(), dW.clone(), db.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_set_weight_twice_replaces_spectra():
    inp1 = make_inputs(32, 64, 300, dtype="f32", seed=1)
    inp2 = make_inputs(32, 64, 300, dtype="f32", seed=2)
    plan = Plan(32, 64, "f32")
    x = to_dev(inp1["x"])
    plan.set_weight(to_dev(inp1["W"]), to_dev(inp1["bias"]))
    plan.set_weight(to_dev(inp2["W"]), to_dev(inp2["bias"]))
    y = plan.forward(x)
    _sync()
    ref = oracle.forward(inp1["x"], inp2["W"], inp2["bias"])
    assert rel_err(to_np64(y), ref) <= TOL["f32"]


# ---- fused activation (forward_act) ------------------------------------------

def _forward_act_case(C, D, N, dtype, act, T=4, seed=0):
    inp = make_inputs(C, D, N, T, dtype=dtype, seed=seed, bias=True)
    plan = Plan(C, D, dtype, T=T)
    plan.set_weight(to_dev(inp["W"]), to_dev(inp["bias"]))
    y = plan.forward(to_dev(inp["x"]), act=act)
    _sync()
    ref = oracle.forward_act(inp["x"], inp["W"], inp["bias"], act)
    err = rel_err(to_np64(y), ref)
    print(f"forward_act {act} T={T} C={C} D={D} N={N} {dtype}: rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype], err
    plan.close()


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh"])
@pytest.mark.parametrize("C,D,N,dtype,env", [
    (96, 384, 3001, "f16", {}),                         # producer/consumer binary16, pipelined epilogue
    (96, 384, 3001, "f16", {"EQL_WS_PIPE": "0"}),       # not pipelined
    (96, 384, 3001, "f16", {"EQL_WS_SMALL_MB": "0"}),   # split stores (outputs beyond the cache)
    (96, 384, 3001, "f16", {"EQL_WS_NC": "4", "EQL_WS_NB": "2"}),  # 4 consumers of 32 channels
    (256, 96, 700, "f16", {}),                          # 8-channel producer units (long reduction)
    (96, 384, 3001, "f32", {}),                         # producer/consumer binary32
    (96, 96, 1000, "f32", {"EQL_WS32_NC": "12"}),       # binary32, reduction split over wave pairs
    (33, 130, 65, "f16", {}),                           # fallback kernel + activation pass
    (33, 130, 65, "f32", {}),
    (96, 96, 1000, "f16", {"EQL_NO_WS": "1"}),          # tiled fallback + activation pass
    (96, 96, 1000, "f32", {"EQL_NO_WS32": "1"}),
])
def test_forward_act(C, D, N, dtype, env, act, monkeypatch):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    _forward_act_case(C, D, N, dtype, act, seed=21)


# ---- seeded random shapes for the weight gradient ---------------------------

def _random_bw_shapes(n, seed=11):
    """(C, D, N, splits) with even channel counts (the producer/consumer
    kernel's domain), row counts that leave ragged 32-row steps and splits
    of odd and even step counts; splits 0 keeps the library's choice."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        C = 2 * int(rng.integers(1, 97))
        D = 2 * int(rng.integers(1, 129))
        N = int(rng.integers(1, 4000))
        out.append((C, D, N, int(rng.choice([0, 1, 2, 3, 5, 9]))))
    return out


@pytest.mark.parametrize("C,D,N,splits", _random_bw_shapes(16))
def test_backward_weight_random_shapes(C, D, N, splits, monkeypatch):
    if splits:
        monkeypatch.setenv("EQL_BWS_S", str(splits))
    inp = make_inputs(C, D, N, dtype="f16", seed=C * 7 + D + N, bias=True, dy=True)
    plan = Plan(C, D, "f16")
    dW, db = plan.backward_weight(to_dev(inp["x"]), to_dev(inp["dy"]))
    _sync()
    ref_dW, ref_db = oracle.backward_weight(inp["x"], inp["dy"])
    e = (rel_err(to_np64(dW), ref_dW), rel_err(to_np64(db), ref_db))
    print(f"backward_weight random C={C} D={D} N={N} splits={splits}: dW {e[0]:.3e} dbias {e[1]:.3e}",
          flush=True)
    assert max(e) <= TOL["f16"], e
    plan.close()
