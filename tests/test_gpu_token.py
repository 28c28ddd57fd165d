"""Token-major activations and outputs (x [N, K] in, c [N, M] out) on every
kernel that takes them, against the oracle element by element, and bit for
bit against the [K, N] layout under the same plan (same products, same
summation order, same rounding)."""

import numpy as np
import pytest

from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import Problem, assert_parity, log, run

pytestmark = pytest.mark.gpu

_probs = {}


def prob(M, K):
    key = (M, K)
    if key not in _probs:
        _probs[key] = Problem(M, K, seed=40 + len(_probs))
    return _probs[key]


def X_for(K, N, seed=0):
    return inputs.activations(K, N, wid=300 + seed, layer=K, proj=N)


def both_layouts(M, K, N, plan, what):
    p = prob(M, K)
    X = X_for(K, N)
    C_tok = run(p, X, plan=plan, layout=B.LAYOUT_TOKEN)
    C_ref, A_ref = p.reference(X)
    assert_parity(C_tok, C_ref, A_ref, what)
    C_kn = run(p, X, plan=plan, layout=B.LAYOUT_KN)
    assert np.array_equal(C_tok.view(np.uint16), C_kn.view(np.uint16)), what + ": layouts differ"


PLANS = [
    # (M, K, N, plan fields): ragged tails in M and N, splits, wave grids
    (1, 128, 1, dict(kernel=1, ncol=1, rb=1, wm=1, wk=1, splitk=1)),
    (130, 4096, 1, dict(kernel=1, ncol=1, rb=1, wm=1, wk=8, splitk=2)),
    (40, 384, 2, dict(kernel=1, ncol=2, rb=1, wm=1, wk=1, splitk=1)),
    (40, 384, 3, dict(kernel=1, ncol=3, rb=1, wm=1, wk=2, splitk=1)),
    (77, 1152, 4, dict(kernel=1, ncol=4, rb=1, wm=2, wk=1, splitk=2)),
    (77, 1152, 5, dict(kernel=1, ncol=5, rb=1, wm=2, wk=2, splitk=1)),
    (77, 1152, 6, dict(kernel=1, ncol=6, rb=1, wm=1, wk=4, splitk=1)),
    (77, 1152, 7, dict(kernel=1, ncol=7, rb=1, wm=1, wk=2, splitk=2)),
    (96, 1152, 8, dict(kernel=1, ncol=8, rb=1, wm=2, wk=2, splitk=3)),
    (300, 384, 3, dict(kernel=1, ncol=3, rb=1, wm=1, wk=1, splitk=1)),
    (33, 11008, 2, dict(kernel=1, ncol=2, rb=1, wm=1, wk=8, splitk=1)),
    (100, 384, 2, dict(kernel=3, ncol=16, pf=8, splitk=1, rb=1, wk=1)),
    (129, 384, 5, dict(kernel=3, ncol=16, pf=16, splitk=1, rb=2, wk=1)),
    (300, 1152, 16, dict(kernel=3, ncol=16, pf=8, splitk=1, rb=2, wk=1)),
    (300, 1152, 13, dict(kernel=3, ncol=16, pf=16, splitk=2, rb=1, wk=1)),
    (257, 4096, 11, dict(kernel=3, ncol=16, pf=16, splitk=3, rb=1, wk=1)),
    (200, 640, 17, dict(kernel=3, ncol=32, pf=16, splitk=2, rb=2, wk=1)),
    (131, 1152, 31, dict(kernel=3, ncol=32, pf=8, splitk=3, rb=2, wk=1)),
    (300, 4096, 16, dict(kernel=3, ncol=16, pf=8, splitk=1, rb=1, wk=4)),
    (250, 1152, 33, dict(kernel=3, ncol=64, pf=16, splitk=2, rb=1, wk=1)),
    (77, 384, 64, dict(kernel=3, ncol=64, pf=8, splitk=1, rb=2, wk=2)),
    (1, 128, 65, dict(kernel=2, bm=128, bn=64, splitk=1, wm=4)),
    (100, 384, 65, dict(kernel=2, bm=128, bn=64, splitk=1, wm=4)),
    (300, 1152, 200, dict(kernel=2, bm=256, bn=64, splitk=3, wm=4)),
    (257, 384, 264, dict(kernel=2, bm=256, bn=128, splitk=1, wm=4)),
    (257, 1152, 264, dict(kernel=2, bm=128, bn=256, splitk=2, wm=2)),
    (520, 640, 520, dict(kernel=2, bm=256, bn=256, splitk=1, wm=2)),
    (64, 256, 77, dict(kernel=2, bm=128, bn=128, splitk=1, wm=4)),
    (129, 384, 130, dict(kernel=2, bm=256, bn=128, splitk=2, wm=4)),   # M % 4 != 0
    (130, 384, 40, dict(kernel=2, bm=128, bn=64, splitk=1, wm=4)),     # M % 4 == 2
    (40, 128, 3, dict(kernel=2, bm=128, bn=64, splitk=1, wm=4)),
    (520, 640, 520, dict(kernel=2, bm=512, bn=128, splitk=1, wm=8, pf=2)),
    (129, 384, 130, dict(kernel=2, bm=512, bn=128, splitk=2, wm=8, pf=2)),   # M % 4 != 0
    (300, 512, 100, dict(kernel=2, bm=256, bn=128, splitk=1, wm=4, pf=2)),
    # [K, N] read in place (N a multiple of 8) against the chunk layout:
    # ragged column tiles, splits, both K-slice forms, the 86-group tail
    (100, 384, 72, dict(kernel=2, bm=128, bn=64, splitk=1, wm=4)),
    (77, 384, 8, dict(kernel=2, bm=128, bn=64, splitk=1, wm=4, pf=2)),
    (300, 1152, 136, dict(kernel=2, bm=96, bn=64, splitk=2, wm=3, pf=2)),
    (97, 1152, 64, dict(kernel=2, bm=96, bn=64, splitk=3, wm=3, pf=1)),
    (129, 4096, 64, dict(kernel=2, bm=128, bn=64, splitk=4, wm=4, pf=2)),
    (257, 1152, 96, dict(kernel=2, bm=128, bn=64, splitk=1, wm=4, wk=2, pf=1)),
    (130, 1152, 200, dict(kernel=2, bm=128, bn=64, splitk=2, wm=4, wk=2, pf=2)),
    (520, 640, 248, dict(kernel=2, bm=128, bn=64, splitk=1, wm=4, pf=2)),
    (64, 11008, 64, dict(kernel=2, bm=128, bn=64, splitk=2, wm=4, pf=2)),
    (257, 1152, 96, dict(kernel=2, bm=128, bn=128, splitk=1, wm=4, wk=2, pf=1)),
    (520, 640, 248, dict(kernel=2, bm=128, bn=128, splitk=1, wm=4, pf=2)),
    (300, 4096, 136, dict(kernel=2, bm=128, bn=128, splitk=3, wm=4, wk=2, pf=1)),
    (513, 1152, 1024, dict(kernel=2, bm=512, bn=128, splitk=1, wm=8, pf=2)),
    (300, 640, 392, dict(kernel=2, bm=256, bn=128, splitk=2, wm=4, pf=1)),
]


@pytest.mark.parametrize("case", PLANS, ids=lambda c: "M%d_K%d_N%d_k%d" % (c[0], c[1], c[2], c[3]["kernel"]))
def test_token_plan(case):
    M, K, N, fields = case
    log("token %s" % (case,))
    both_layouts(M, K, N, B.Plan.make(**fields), str(case))


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 17, 31, 32, 33, 64, 100, 256])
def test_token_default_dispatch(N):
    M, K = 333, 1152
    log("token default N=%d" % N)
    p = prob(M, K)
    X = X_for(K, N, seed=1)
    C = run(p, X, layout=B.LAYOUT_TOKEN)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, "token default N=%d" % N)


@pytest.mark.parametrize("N", [1, 4, 16, 32, 128])
def test_token_default_full_rows(N):
    """The 12288 x 4096 projection at decode and small-prefill widths,
    checked on sampled rows (the oracle computes them one by one)."""
    M, K = 12288, 4096
    log("token full M=%d K=%d N=%d" % (M, K, N))
    p = prob(M, K)
    X = X_for(K, N, seed=2)
    C = run(p, X, layout=B.LAYOUT_TOKEN)
    rows = np.random.default_rng(N).choice(M, 64, replace=False)
    C_ref, A_ref = p.reference_rows(X, rows)
    assert_parity(C[rows], C_ref, A_ref, "token full N=%d" % N)
