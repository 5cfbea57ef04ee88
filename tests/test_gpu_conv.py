"""GPU parity of the p4 group convolution (include/eqconv.h) against the fp64
oracle, through the C ABI: forward (with and without the fused GELU),
backward input and backward filter, on ragged pixel counts, kernel sizes 1, 3
and 5, both tile shapes, degenerate images, equivariance on the device, and
the full Swin-like stage shape over every output of the three passes."""
import numpy as np
import pytest

import oracle
from group_dft_structured_amd import ConvPlan, EqlinearError
from group_dft_structured_amd.workloads import CONV_WORKLOADS, make_conv_inputs
from tests.gpu_helpers import TOL, gpu_available, rel_err, to_dev, to_np64, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


# (N, H, W, C, D, k): pixel counts off the 16- and 64-pixel tiles, output
# widths on both LDS tile shapes (D <= 64 and D > 64), patch widths of
# several steps with a ragged last one, kernel sizes 1, 3 and 5, non-square
# images.  Patch widths of 4 to 24 reduction steps run the register-direct
# binary16 kernel (every variant of it: 1 to 6 steps per wave, three or two
# channel blocks per work-group); the others the LDS-tiled one.
SHAPES = [
    (2, 7, 9, 8, 12, 3),
    (1, 13, 11, 4, 68, 3),
    (2, 6, 5, 16, 8, 5),
    (3, 4, 4, 12, 4, 1),
    (1, 20, 20, 32, 40, 3),
    (1, 9, 12, 20, 132, 3),
    (1, 10, 9, 64, 40, 3),
    (1, 6, 7, 128, 20, 3),
    (1, 7, 6, 12, 24, 3),
    (1, 5, 6, 80, 16, 3),
]


def _case(shape, dtype, seed=5, bias=True):
    N, H, W, C, D, k = shape
    inp = make_conv_inputs(N, H, W, C, D, k, dtype=dtype, seed=seed, bias=bias, dy=True)
    plan = ConvPlan(C, D, k, dtype)
    plan.set_weight(to_dev(inp["psi"]), to_dev(inp["bias"]))
    return inp, plan


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward(shape, dtype):
    inp, plan = _case(shape, dtype)
    y = plan.forward(to_dev(inp["f"]))
    ref = oracle.conv_forward(inp["f"], inp["psi"], inp["bias"])
    assert rel_err(to_np64(y), ref) <= TOL[dtype]
    plan.close()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("act", ["gelu", "gelu_tanh"])
def test_forward_act(act, dtype):
    inp, plan = _case((2, 7, 9, 8, 12, 3), dtype)
    y = plan.forward(to_dev(inp["f"]), act=act)
    ref = oracle.conv_forward_act(inp["f"], inp["psi"], inp["bias"], act)
    assert rel_err(to_np64(y), ref) <= TOL[dtype]
    plan.close()


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh"])
@pytest.mark.parametrize("shape", [(2, 7, 9, 48, 48, 3), (1, 10, 9, 64, 40, 3), (1, 9, 12, 20, 132, 3)],
                         ids=lambda s: "x".join(map(str, s)))
def test_forward_act_register_direct(shape, act):
    """The fused activation on the register-direct binary16 kernel, whose
    host split of the reduction steps depends on the activation: 14, 18 and
    6 steps, channel counts 48 and 64 (wave-uniform orbit addressing) and 20
    (per-lane addressing)."""
    inp, plan = _case(shape, "f16")
    y = plan.forward(to_dev(inp["f"]), act=act)
    ref = oracle.conv_forward_act(inp["f"], inp["psi"], inp["bias"], act)
    assert rel_err(to_np64(y), ref) <= TOL["f16"]
    plan.close()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_input(shape, dtype):
    inp, plan = _case(shape, dtype)
    df = plan.backward_input(to_dev(inp["dy"]))
    ref = oracle.conv_backward_input(inp["dy"], inp["psi"])
    assert rel_err(to_np64(df), ref) <= TOL[dtype]
    plan.close()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_weight(shape, dtype):
    inp, plan = _case(shape, dtype)
    dpsi, dbias = plan.backward_weight(to_dev(inp["f"]), to_dev(inp["dy"]))
    rpsi, rbias = oracle.conv_backward_weight(inp["f"], inp["dy"], shape[5])
    assert rel_err(to_np64(dpsi), rpsi) <= TOL[dtype]
    assert rel_err(to_np64(dbias), rbias) <= TOL[dtype]
    plan.close()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_equivariance_on_device(dtype):
    """Turning the input a quarter turn with the group shift turns the output
    the same way; compared on the device outputs themselves."""
    torch = torch_mod()
    inp, plan = _case((2, 10, 10, 8, 12, 3), dtype)
    f = to_dev(inp["f"])
    y = plan.forward(f)
    for r in (1, 2, 3):
        fr = torch.roll(torch.rot90(f, r, dims=(1, 2)), r, dims=4).contiguous()
        yr = plan.forward(fr)
        want = torch.roll(torch.rot90(y, r, dims=(1, 2)), r, dims=4)
        assert rel_err(to_np64(yr), to_np64(want)) <= TOL[dtype], r
    plan.close()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_degenerate_images(dtype):
    """Single-row, single-column and single-pixel images: every neighbour of
    some pixels lies outside the image."""
    for shape in [(3, 1, 9, 8, 8, 3), (2, 7, 1, 8, 8, 3), (5, 1, 1, 8, 8, 5)]:
        inp, plan = _case(shape, dtype)
        y = plan.forward(to_dev(inp["f"]))
        assert rel_err(to_np64(y), oracle.conv_forward(inp["f"], inp["psi"], inp["bias"])) \
            <= TOL[dtype], shape
        df = plan.backward_input(to_dev(inp["dy"]))
        assert rel_err(to_np64(df), oracle.conv_backward_input(inp["dy"], inp["psi"])) \
            <= TOL[dtype], shape
        plan.close()


def test_zero_pixels_and_errors():
    torch = torch_mod()
    inp, plan = _case((2, 4, 4, 8, 8, 3), "f32")
    y = torch.empty((0, 4, 4, 8, 4), device="cuda")
    plan.forward(torch.empty((0, 4, 4, 8, 4), device="cuda"), y)
    dpsi, dbias = plan.backward_weight(torch.empty((2, 0, 4, 8, 4), device="cuda"),
                                       torch.empty((2, 0, 4, 8, 4), device="cuda"))
    torch.cuda.synchronize()
    assert float(dpsi.abs().max()) == 0.0 and float(dbias.abs().max()) == 0.0
    fresh = ConvPlan(8, 8, 3, "f32")
    with pytest.raises(EqlinearError):
        fresh.forward(to_dev(inp["f"]))  # no weight set
    fresh.close()
    plan.close()


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_stage_shape_full(dtype):
    """The Swin-like stage shape (64 images at 56 x 56, 48 -> 48 channels,
    3 x 3) in the launch configuration the benchmark times, every output of
    the three passes against the oracle: forward and backward input over all
    images (the oracle in chunks of 16 images), the filter gradient with the
    real upstream gradient of every image (the full-size split reduction)."""
    w = CONV_WORKLOADS["p4conv_stage"]
    inp = make_conv_inputs(w.N, w.H, w.W, w.C, w.D, w.k, dtype=dtype, seed=0, bias=True, dy=True)
    plan = ConvPlan(w.C, w.D, w.k, dtype)
    plan.set_weight(to_dev(inp["psi"]), to_dev(inp["bias"]))
    f, dy = to_dev(inp["f"]), to_dev(inp["dy"])
    y = plan.forward(f)
    df = plan.backward_input(dy)
    dpsi, dbias = plan.backward_weight(f, dy)
    torch_mod().cuda.synchronize()

    def blocked(got, ref_fn, chunk=16):
        err_max = ref_max = 0.0
        for i0 in range(0, w.N, chunk):
            ref = ref_fn(slice(i0, i0 + chunk))
            err_max = max(err_max, float(np.abs(to_np64(got[i0:i0 + chunk]) - ref).max()))
            ref_max = max(ref_max, float(np.abs(ref).max()))
        return err_max / ref_max

    e_y = blocked(y, lambda sl: oracle.conv_forward(inp["f"][sl], inp["psi"], inp["bias"]))
    e_df = blocked(df, lambda sl: oracle.conv_backward_input(inp["dy"][sl], inp["psi"]))
    rpsi, rbias = oracle.conv_backward_weight(inp["f"], inp["dy"], w.k)
    e_w, e_b = rel_err(to_np64(dpsi), rpsi), rel_err(to_np64(dbias), rbias)
    print(f"p4conv_stage {dtype}: y {e_y:.3e} df {e_df:.3e} dpsi {e_w:.3e} dbias {e_b:.3e}",
          flush=True)
    for e in (e_y, e_df, e_w, e_b):
        assert e <= TOL[dtype], (e_y, e_df, e_w, e_b)
    plan.close()


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_determinism_bitwise(dtype):
    """Repeat calls give bit-identical results: the reductions (over patch
    channels inside a tile, over pixel splits for the filter gradient) run in
    a fixed order."""
    torch = torch_mod()
    inp, plan = _case((2, 21, 19, 48, 48, 3), dtype)
    f, dy = to_dev(inp["f"]), to_dev(inp["dy"])
    first = [plan.forward(f), plan.backward_input(dy), *plan.backward_weight(f, dy)]
    for _ in range(2):
        again = [plan.forward(f), plan.backward_input(dy), *plan.backward_weight(f, dy)]
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)
    plan.close()


@pytest.mark.parametrize("dtype,env", [("f16", "EQL_CONV_RD"), ("f32", "EQL_CONV_F32_16")])
def test_lds_tiled_kernel_on_default_shapes(monkeypatch, dtype, env):
    """The LDS-tiled kernel (32x32 matrix-core steps) also serves the shapes
    whose default is the register-direct (binary16) or 16x16x4 (binary32)
    kernel when those are switched off; it stays at the oracle bar there."""
    monkeypatch.setenv(env, "0")
    for shape in [(2, 7, 9, 48, 48, 3), (1, 9, 12, 20, 132, 3)]:
        inp, plan = _case(shape, dtype)
        y = plan.forward(to_dev(inp["f"]))
        assert rel_err(to_np64(y), oracle.conv_forward(inp["f"], inp["psi"], inp["bias"])) \
            <= TOL[dtype], shape
        df = plan.backward_input(to_dev(inp["dy"]))
        assert rel_err(to_np64(df), oracle.conv_backward_input(inp["dy"], inp["psi"])) \
            <= TOL[dtype], shape
        plan.close()


def _random_shapes(n, seed=7):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        k = int(rng.choice([1, 3, 5, 7]))
        C = 4 * int(rng.integers(1, 25))
        D = 4 * int(rng.integers(1, 41))
        H, W = int(rng.integers(1, 14)), int(rng.integers(1, 14))
        out.append((int(rng.integers(1, 3)), H, W, C, D, k))
    return out


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_random_shapes(dtype):
    """Seeded random shapes across every kernel and split the library picks
    (kernel sizes 1 to 7, channel counts 4 to 160, images 1 to 13 wide)."""
    for shape in _random_shapes(14):
        inp, plan = _case(shape, dtype, seed=11)
        y = plan.forward(to_dev(inp["f"]))
        assert rel_err(to_np64(y), oracle.conv_forward(inp["f"], inp["psi"], inp["bias"])) \
            <= TOL[dtype], shape
        df = plan.backward_input(to_dev(inp["dy"]))
        assert rel_err(to_np64(df), oracle.conv_backward_input(inp["dy"], inp["psi"])) \
            <= TOL[dtype], shape
        dpsi, db = plan.backward_weight(to_dev(inp["f"]), to_dev(inp["dy"]))
        rpsi, rb = oracle.conv_backward_weight(inp["f"], inp["dy"], shape[5])
        assert rel_err(to_np64(dpsi), rpsi) <= TOL[dtype], shape
        assert rel_err(to_np64(db), rb) <= TOL[dtype], shape
        plan.close()
