"""Exact structural cases on the GPU, for every kernel: q == z gives 0,
identity activation columns recover single dequantized weights, and the
constant case gives 4096 * 15 * fp16(0.02) = 1229.0625 (1229.0 in fp16).
These catch indexing mistakes that random inputs under the loose tolerance
can hide (a dropped group, a shifted scale or zero)."""

import numpy as np
import pytest

from gemm_w4a16_group_amd import binding as B
from gpu_util import Problem, assert_parity, log, run

pytestmark = pytest.mark.gpu

PLANS = [
    ("default", None),
    ("skinny_c1_wk4", B.Plan.make(kernel=1, ncol=1, rb=1, wm=1, wk=4, splitk=1)),
    ("skinny_c16_split", B.Plan.make(kernel=1, ncol=16, rb=1, wm=2, wk=4, splitk=4)),
    ("skinny_c32", "c32"),
    ("tiled_256", B.Plan.make(kernel=2, bm=256, bn=256, splitk=1)),
    ("tiled_128x64_split", B.Plan.make(kernel=2, bm=128, bn=64, splitk=2)),
]


def _plan(plan, K):
    if plan == "c32":   # 32 staged columns: at most two groups (16 KB of LDS) per wave
        G = K // 128
        return B.Plan.make(kernel=1, ncol=32, rb=1, wm=1, wk=2, splitk=(G + 3) // 4)
    return plan


def _ncols(plan, want):
    # a skinny plan is built for exactly plan.ncol activation columns
    if plan is not None and plan.kernel == B.KERNEL_SKINNY:
        return plan.ncol
    return want


@pytest.mark.parametrize("name,plan", PLANS, ids=[p[0] for p in PLANS])
def test_q_equals_z(name, plan):
    M, K = 160, 4096
    plan = _plan(plan, K)
    G = K // 128
    rng = np.random.default_rng(5)
    z = rng.integers(0, 16, (M, G), dtype=np.uint8)
    q = np.repeat(z, 128, axis=1)
    s = rng.uniform(0.002, 0.02, (M, G)).astype(np.float16)
    p = Problem(M, K, q=q, s=s, z=z)
    N = _ncols(plan, 16)
    X = rng.standard_normal((K, N)).astype(np.float16)
    log("q==z %s" % name)
    C = run(p, X, plan=plan)
    assert np.all(np.abs(C.astype(np.float64)) <= 1e-3), np.abs(C).max()


@pytest.mark.parametrize("name,plan", PLANS, ids=[p[0] for p in PLANS])
def test_identity_columns(name, plan):
    M, K = 200, 1152
    plan = _plan(plan, K)
    p = Problem(M, K, seed=9)
    ks = [0, 7, 8, 127, 128, 129, 255, 640, K - 1, 1000, 31, 32, 33, 64, 96, 1151 - 8]
    N = _ncols(plan, len(ks))
    ks = (ks + [int(k) for k in np.random.default_rng(11).integers(0, K, N)])[:N]
    X = np.zeros((K, N), dtype=np.float16)
    for n, k in enumerate(ks):
        X[k, n] = 1.0
    log("identity %s" % name)
    C = run(p, X, plan=plan)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, "identity " + name)
    # each column must be the fp16 rounding of a single dequantized weight
    # (the tiled kernel rounds (q - z) * s to fp16 first; both agree here)
    want = C_ref.astype(np.float16)
    assert np.array_equal(C.view(np.uint16), want.view(np.uint16)), name


@pytest.mark.parametrize("name,plan", PLANS, ids=[p[0] for p in PLANS])
def test_constant_closed_form(name, plan):
    M, K = 96, 4096
    plan = _plan(plan, K)
    G = K // 128
    q = np.full((M, K), 15, dtype=np.uint8)
    z = np.zeros((M, G), dtype=np.uint8)
    s = np.full((M, G), 0.02, dtype=np.float16)
    p = Problem(M, K, q=q, s=s, z=z)
    N = _ncols(plan, 4)
    X = np.ones((K, N), dtype=np.float16)
    log("constant %s" % name)
    C = run(p, X, plan=plan)
    assert np.all(C == np.float16(1229.0625)), np.unique(C)
