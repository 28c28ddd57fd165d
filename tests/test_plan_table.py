"""The plan table's bookkeeping on the CPU: keys, JSON round trip, refusal
of malformed files, and that a recorded plan is one the library accepts."""

import ctypes

import pytest

from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd.plans import PlanTable


def test_round_trip_and_lookup(tmp_path):
    t = PlanTable()
    p = B.Plan.make(kernel=B.KERNEL_TILED, bm=256, bn=128, wm=4, splitk=1)
    t.put(12288, 4096, 4096, B.LAYOUT_KN, p, 452.0)
    q = B.Plan.make(kernel=B.KERNEL_SKINNY, ncol=1, rb=1, wm=1, wk=8, splitk=1)
    t.put(12288, 1, 4096, B.LAYOUT_TOKEN, q, 7.3)
    assert len(t) == 2
    assert t.plan(12288, 4096, 4096).as_dict() == p.as_dict()
    assert t.plan(12288, 1, 4096, B.LAYOUT_TOKEN).as_dict() == q.as_dict()
    assert t.plan(12288, 1, 4096, B.LAYOUT_KN) is None
    path = tmp_path / "plans.json"
    t.save(str(path))
    u = PlanTable.load(str(path))
    assert u.to_json() == t.to_json()
    # every recorded plan is valid for its shape
    lib = B.load_library()
    for M, N, K, plan in ((12288, 4096, 4096, p), (12288, 1, 4096, q)):
        assert lib.w4a16_kernel_name(M, N, K, 128, ctypes.byref(plan), ctypes.create_string_buffer(64), 64) == 0


@pytest.mark.parametrize("text", ['{"plans": {}}', '{"w4a16_plan_table": 1, "plans": {"1,2,3": {"plan": {}}}}',
                                  '{"w4a16_plan_table": 1, "plans": {"1,2,3,0": {"plan": {"kernel": 1}}}}'])
def test_malformed_tables_are_refused(text):
    with pytest.raises(ValueError):
        PlanTable.from_json(text)
