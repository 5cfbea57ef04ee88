"""eqlinear_backward_weight_noalloc (the weight gradient without a workspace
argument or any device allocation) against eqlinear_backward_weight on the
same inputs, through the C ABI: bit-identical results (same kernels, same
fixed reduction order) and within the oracle bar, on two calls in a row, the
second with fewer rows, for every kernel family that takes a workspace."""
import numpy as np
import pytest

import oracle
from group_dft_structured_amd import (EQL_F16, EQL_F32, EQL_GROUP_CYCLIC, EQL_GROUP_DIHEDRAL,
                                      eqlinear_backward_weight, eqlinear_backward_weight_noalloc,
                                      eqlinear_backward_weight_workspace,
                                      eqlinear_plan_create_group, eqlinear_plan_destroy,
                                      eqlinear_set_weight)
from group_dft_structured_amd.workloads import make_inputs
from tests.gpu_helpers import TOL, gpu_available, rel_err, to_dev, to_np64, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


# (group, n, T, dtype, C, D, first N, second N): the p4 producer/consumer
# kernel at the ViT-S MLP backward shape, the tiled kernel (binary32, odd
# widths), the generic cyclic kernels and p4m on paired p4 channels
CASES = [
    (EQL_GROUP_CYCLIC, 4, 4, "f16", 96, 384, 12608, 3001),
    (EQL_GROUP_CYCLIC, 4, 4, "f32", 33, 70, 2000, 517),
    (EQL_GROUP_CYCLIC, 8, 8, "f16", 48, 192, 4000, 999),
    (EQL_GROUP_DIHEDRAL, 4, 8, "f16", 48, 64, 3000, 100),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"g{c[0]}n{c[1]}-{c[3]}-{c[4]}x{c[5]}")
def test_noalloc_matches_workspace_entry_point(case):
    torch = torch_mod()
    group, n, T, dtype, C, D, N1, N2 = case
    code = EQL_F16 if dtype == "f16" else EQL_F32
    plan = eqlinear_plan_create_group(C, D, group, n, code)
    gname = "cyclic" if group == EQL_GROUP_CYCLIC else "dihedral"
    try:
        for N in (N1, N2):
            inp = make_inputs(C, D, N, T, dtype=dtype, seed=N, bias=True, dy=True)
            eqlinear_set_weight(plan, to_dev(inp["W"]), to_dev(inp["bias"]))
            x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
            need = eqlinear_backward_weight_workspace(plan, N)
            ws = torch.empty((max(need, 16),), dtype=torch.uint8, device="cuda")
            dW_ref = torch.empty((D, C, T), dtype=torch.float32, device="cuda")
            db_ref = torch.empty((D,), dtype=torch.float32, device="cuda")
            eqlinear_backward_weight(plan, x, dy, dW_ref, db_ref, N, ws, ws.numel())
            dW = torch.full((D, C, T), 7.0, dtype=torch.float32, device="cuda")
            db = torch.full((D,), 7.0, dtype=torch.float32, device="cuda")
            eqlinear_backward_weight_noalloc(plan, x, dy, dW, db, N)
            torch.cuda.synchronize()
            print(f"noalloc {gname} T={T} {dtype} C={C} D={D} N={N}: workspace {need} B",
                  flush=True)
            assert torch.equal(dW, dW_ref) and torch.equal(db, db_ref)
            ref_dW, ref_db = oracle.backward_weight(inp["x"], inp["dy"], group=gname)
            assert rel_err(to_np64(dW), ref_dW) <= TOL[dtype]
            assert rel_err(to_np64(db), ref_db) <= TOL[dtype]
    finally:
        eqlinear_plan_destroy(plan)


def test_noalloc_zero_rows_writes_zeros():
    torch = torch_mod()
    plan = eqlinear_plan_create_group(16, 16, EQL_GROUP_CYCLIC, 4, EQL_F16)
    try:
        x = torch.empty((0, 16, 4), dtype=torch.float16, device="cuda")
        dW = torch.full((16, 16, 4), 7.0, device="cuda")
        db = torch.full((16,), 7.0, device="cuda")
        eqlinear_backward_weight_noalloc(plan, x, x, dW, db, 0)
        torch.cuda.synchronize()
        assert float(dW.abs().max()) == 0.0 and float(db.abs().max()) == 0.0
    finally:
        eqlinear_plan_destroy(plan)
