"""A per-shape plan table: the tuner's choices, kept and reused.

`PlanTable.tune()` runs the library's tuner (`w4a16_tune`, timed on the
device with the caller's buffers) for one call shape and records the
winner under (M, N, K, layout); `plan()` returns the recorded plan or None
(None lets the library use its built-in default).  A table saves to and
loads from JSON, so a sweep over N done once (the N thresholds and tile
sizes of one projection) serves later runs.  Only host bookkeeping lives
here; every product runs in the library's kernels.
"""

import json

from . import binding as B


class PlanTable:
    def __init__(self):
        self._plans = {}

    @staticmethod
    def _key(M, N, K, layout):
        return "%d,%d,%d,%d" % (M, N, K, layout)

    def __len__(self):
        return len(self._plans)

    def plan(self, M, N, K, layout=B.LAYOUT_KN):
        rec = self._plans.get(self._key(M, N, K, layout))
        return None if rec is None else B.Plan.make(**rec["plan"])

    def put(self, M, N, K, layout, plan, us=None):
        self._plans[self._key(M, N, K, layout)] = {"plan": plan.as_dict(), "us": us}

    def tune(self, qpk, s, zpk, x, layout=B.LAYOUT_KN, iters=10, flush=None):
        """Tune this call's shape and record the result; returns the plan."""
        M, N, K = B._dims(qpk, s, zpk, x, layout)
        plan, us, _ = B.tune(qpk, s, zpk, x, layout=layout, iters=iters, flush=flush)
        self.put(M, N, K, layout, plan, us)
        return plan

    def gemm(self, qpk, s, zpk, x, out=None, layout=B.LAYOUT_KN, workspace=None):
        """binding.gemm with this table's plan for the shape (the library's
        default when the shape was never tuned)."""
        M, N, K = B._dims(qpk, s, zpk, x, layout)
        return B.gemm(qpk, s, zpk, x, out=out, plan=self.plan(M, N, K, layout), workspace=workspace,
                      layout=layout)

    def to_json(self):
        return json.dumps({"w4a16_plan_table": 1, "plans": self._plans}, indent=1, sort_keys=True)

    @classmethod
    def from_json(cls, text):
        data = json.loads(text)
        if data.get("w4a16_plan_table") != 1:
            raise ValueError("not a w4a16 plan table")
        t = cls()
        fields = {f for f, _ in B.Plan._fields_}
        for key, rec in data["plans"].items():
            parts = key.split(",")
            if len(parts) != 4 or not all(p.lstrip("-").isdigit() for p in parts):
                raise ValueError("bad plan key %r" % key)
            plan = rec["plan"]
            if set(plan) != fields:
                raise ValueError("plan %r has fields %s" % (key, sorted(plan)))
            t._plans[key] = {"plan": {k: int(v) for k, v in plan.items()}, "us": rec.get("us")}
        return t

    def save(self, path):
        with open(path, "w") as f:
            f.write(self.to_json())

    @classmethod
    def load(cls, path):
        with open(path) as f:
            return cls.from_json(f.read())
