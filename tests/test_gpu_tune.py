"""The plan tuner: it times several plans, returns one the shape admits, and
that plan's results meet the parity rule, for both layouts and each
kernel family's range of N."""

import pytest
import torch

from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import Problem, assert_parity, dev, log, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [1, 4, 16, 40, 200])
@pytest.mark.parametrize("layout", [B.LAYOUT_KN, B.LAYOUT_TOKEN], ids=["kn", "token"])
def test_tuned_plan_is_valid_and_correct(N, layout):
    M, K = 300, 1152
    log("tune N=%d layout=%d" % (N, layout))
    p = Problem(M, K, seed=70 + N)
    X = inputs.activations(K, N, wid=700 + N)
    xd = dev(X.T if layout == B.LAYOUT_TOKEN else X)
    flush = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    plan, us, tried = B.tune(p.qpk, p.s_d, p.zpk, xd, layout=layout, iters=3, flush=flush)
    assert tried > 1 and us > 0
    assert plan.kernel in (B.KERNEL_SKINNY, B.KERNEL_NARROW, B.KERNEL_TILED)
    C = run(p, X, plan=plan, layout=layout)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, "tuned N=%d %s" % (N, plan.as_dict()))


def test_plan_table_tunes_and_serves(tmp_path):
    """A tuned table entry round-trips through JSON and drives gemm()."""
    from gemm_w4a16_group_amd.plans import PlanTable
    M, K, N = 300, 1152, 24
    p = Problem(M, K, seed=90)
    X = inputs.activations(K, N, wid=790)
    t = PlanTable()
    t.tune(p.qpk, p.s_d, p.zpk, dev(X), iters=2)
    path = tmp_path / "plans.json"
    t.save(str(path))
    u = PlanTable.load(str(path))
    assert u.plan(M, N, K) is not None
    C = u.gemm(p.qpk, p.s_d, p.zpk, dev(X))
    torch.cuda.synchronize()
    C_ref, A_ref = p.reference(X)
    assert_parity(C.cpu().numpy(), C_ref, A_ref, "plan table")
