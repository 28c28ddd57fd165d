"""Shapes at the edges of the default dispatch: a single row, very long rows
(many groups: waves along K and splits across workgroups), many rows with
the shortest K, and very many columns, in both layouts."""

import numpy as np
import pytest

from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import Problem, assert_parity, log, run

pytestmark = pytest.mark.gpu

SHAPES = [
    # (M, K, N)
    (1, 128, 1),
    (1, 262144, 1),
    (33, 1048576, 1),
    (64, 131072, 1),
    (64, 65536, 16),
    (70000, 128, 1),
    (70000, 128, 3),
    (100, 128, 30000),
    (5, 640, 5000),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "M%d_K%d_N%d" % s)
@pytest.mark.parametrize("layout", [B.LAYOUT_KN, B.LAYOUT_TOKEN], ids=["kn", "token"])
def test_extreme_shape(shape, layout):
    M, K, N = shape
    log("extreme %s layout %d" % (shape, layout))
    p = Problem(M, K, seed=500 + (M % 97) + N)
    X = inputs.activations(K, N, wid=1200 + N, layer=K)
    C = run(p, X, layout=layout)
    if M * N <= 2_000_000:
        C_ref, A_ref = p.reference(X)
        assert_parity(C, C_ref, A_ref, "%s" % (shape,))
    else:
        rows = np.random.default_rng(M).choice(M, min(M, 32), replace=False)
        C_ref, A_ref = p.reference_rows(X, rows)
        assert_parity(C[rows], C_ref, A_ref, "%s rows" % (shape,))
