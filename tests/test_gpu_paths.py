"""Every kernel variant against the oracle on small, ragged shapes: several
tiles, tails in M and N, every activation staging width, every split.
Element-by-element, with the rule |C - C_ref| <= 5e-3 * sum|W X| + 1e-3."""

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
        _probs[key] = Problem(M, K, seed=len(_probs))
    return _probs[key]


def X_for(K, N, seed=0):
    return inputs.activations(K, N, wid=200 + seed, layer=K, proj=N)


SKINNY = [
    # (M, K, N, ncol, rb, wm, wk, splitk); ncol == N (the kernel is built
    # per column count: 1..8, 16, 32) and rb == 1
    (1, 128, 1, 1, 1, 1, 1, 1),
    (17, 384, 1, 1, 1, 1, 2, 1),
    (63, 1152, 1, 1, 1, 1, 4, 1),
    (200, 1152, 1, 1, 1, 2, 4, 1),
    (200, 1152, 1, 1, 1, 2, 2, 3),
    (130, 4096, 1, 1, 1, 1, 8, 2),
    (130, 4096, 1, 1, 1, 1, 2, 1),
    (33, 11008, 1, 1, 1, 1, 8, 1),
    (33, 11008, 1, 1, 1, 1, 16, 1),
    (33, 11008, 1, 1, 1, 2, 8, 3),
    (40, 384, 2, 2, 1, 1, 1, 1),
    (40, 384, 3, 3, 1, 1, 2, 1),
    (77, 1152, 4, 4, 1, 2, 1, 2),
    (77, 1152, 5, 5, 1, 2, 2, 1),
    (77, 1152, 6, 6, 1, 1, 4, 1),
    (77, 1152, 7, 7, 1, 1, 2, 2),
    (96, 1152, 8, 8, 1, 2, 2, 3),
    (96, 1152, 8, 8, 1, 2, 4, 1),
    (130, 1152, 16, 16, 1, 1, 4, 2),
    (130, 1152, 16, 16, 1, 1, 4, 1),
    (64, 1152, 32, 32, 1, 1, 4, 3),
    (64, 1152, 32, 32, 1, 2, 2, 5),
    (50, 640, 32, 32, 1, 1, 2, 3),
    (50, 640, 32, 32, 1, 2, 1, 5),
    (300, 384, 2, 2, 1, 1, 1, 1),
    (300, 384, 3, 3, 1, 1, 1, 1),
]


@pytest.mark.parametrize("case", SKINNY, ids=lambda c: "M%d_K%d_N%d_c%d_rb%d_wm%d_wk%d_s%d" % c)
def test_skinny_plan(case):
    M, K, N, ncol, rb, wm, wk, splitk = case
    log("skinny %s" % (case,))
    p = prob(M, K)
    X = X_for(K, N)
    plan = B.Plan.make(kernel=B.KERNEL_SKINNY, ncol=ncol, rb=rb, wm=wm, wk=wk, splitk=splitk)
    C = run(p, X, plan=plan)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, str(case))


TILED = [
    # (M, K, N, bm, bn, splitk, wm)
    (1, 128, 65, 128, 64, 1, 4),
    (100, 384, 65, 128, 64, 1, 4),
    (300, 384, 100, 128, 128, 1, 4),
    (300, 1152, 128, 128, 64, 2, 4),
    (300, 1152, 200, 256, 64, 3, 4),
    (257, 384, 264, 256, 128, 1, 4),
    (257, 1152, 264, 128, 256, 2, 4),
    (520, 640, 520, 256, 256, 1, 4),
    (520, 640, 256, 256, 256, 4, 4),
    (64, 256, 77, 128, 128, 1, 4),       # N not a multiple of 8
    (129, 384, 130, 256, 128, 2, 4),
    (40, 128, 3, 128, 64, 1, 4),         # small N on the tiled kernel
    # 2 x 2 wave grid
    (300, 384, 100, 128, 128, 1, 2),
    (257, 1152, 264, 128, 256, 2, 2),
    (520, 640, 520, 256, 256, 1, 2),
    (129, 384, 130, 256, 128, 2, 2),
]


@pytest.mark.parametrize("case", TILED, ids=lambda c: "M%d_K%d_N%d_bm%d_bn%d_s%d_wm%d" % c)
def test_tiled_plan(case):
    M, K, N, bm, bn, splitk, wm = case
    log("tiled %s" % (case,))
    p = prob(M, K)
    X = X_for(K, N)
    plan = B.Plan.make(kernel=B.KERNEL_TILED, bm=bm, bn=bn, splitk=splitk, wm=wm)
    C = run(p, X, plan=plan)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, str(case))


TILED_DEEP = [
    # (M, K, N, bm, bn, splitk, wm, pf): eight-wave 512-row tiles and weights
    # two stages ahead; group counts that leave 0, 1 or 2 stages after the
    # last whole round of three (1, 2, 3, 4, 5, 9 and 86 groups), splits of
    # uneven length, ragged M and N
    (1, 128, 1, 512, 128, 1, 8, 2),
    (129, 256, 77, 128, 128, 1, 4, 2),
    (513, 384, 130, 512, 128, 1, 8, 2),
    (300, 512, 100, 256, 128, 1, 4, 2),
    (1030, 640, 257, 512, 128, 1, 8, 0),
    (1030, 640, 257, 512, 128, 1, 8, 2),
    (700, 1152, 200, 512, 128, 2, 8, 2),
    (700, 1152, 200, 512, 128, 4, 8, 2),
    (257, 1152, 264, 128, 64, 3, 4, 2),
    (520, 896, 520, 256, 256, 1, 4, 2),
    (64, 11008, 65, 512, 128, 1, 8, 2),
    # 96-row tiles of three waves: ragged M and N, uneven splits, K = 11008
    (1, 128, 65, 96, 64, 1, 3, 1),
    (97, 384, 100, 96, 64, 1, 3, 2),
    (300, 1152, 64, 96, 64, 3, 3, 2),
    (193, 11008, 48, 96, 64, 2, 3, 2),
    (1000, 4096, 128, 96, 64, 2, 3, 1),
]


@pytest.mark.parametrize("case", TILED_DEEP, ids=lambda c: "M%d_K%d_N%d_bm%d_bn%d_s%d_wm%d_pf%d" % c)
def test_tiled_deep_plan(case):
    M, K, N, bm, bn, splitk, wm, pf = case
    log("tiled deep %s" % (case,))
    p = prob(M, K)
    X = X_for(K, N)
    plan = B.Plan.make(kernel=B.KERNEL_TILED, bm=bm, bn=bn, splitk=splitk, wm=wm, pf=pf)
    C = run(p, X, plan=plan)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, str(case))
    # how far ahead the weights are loaded and how many rows a tile has
    # change no arithmetic: the same as 128-row tiles of four waves
    base = B.Plan.make(kernel=B.KERNEL_TILED, bm=128, bn=bn if bn != 256 else 128, splitk=splitk, wm=4)
    assert np.array_equal(C, run(p, X, plan=base)), case


TILED_PIPE = [
    # (M, K, N, bm, bn, splitk, pf, xpf): weights pf and activations xpf
    # stages ahead; fewer stages than the pipeline is deep (1, 2, 3 groups),
    # uneven splits, one stage per split (splitk = G), the 86-group tail,
    # ragged M and N
    (1, 128, 1, 128, 64, 1, 4, 3),
    (129, 256, 77, 128, 64, 1, 2, 2),
    (300, 384, 64, 128, 64, 1, 4, 2),
    (300, 640, 100, 128, 64, 2, 4, 3),
    (257, 1152, 128, 128, 128, 3, 3, 2),
    (257, 1152, 130, 128, 128, 2, 2, 2),
    (520, 4096, 64, 256, 64, 4, 3, 2),
    (200, 11008, 70, 128, 64, 3, 4, 3),
    (1000, 4096, 130, 128, 64, 3, 4, 2),
    (64, 1152, 40, 128, 64, 9, 4, 3),
    (333, 2048, 96, 256, 64, 2, 2, 2),
]


@pytest.mark.parametrize("case", TILED_PIPE, ids=lambda c: "M%d_K%d_N%d_bm%d_bn%d_s%d_pf%d_xpf%d" % c)
def test_tiled_pipeline_plan(case):
    M, K, N, bm, bn, splitk, pf, xpf = case
    log("tiled pipeline %s" % (case,))
    p = prob(M, K)
    X = X_for(K, N)
    plan = B.Plan.make(kernel=B.KERNEL_TILED, bm=bm, bn=bn, splitk=splitk, wm=4, pf=pf, xpf=xpf)
    C = run(p, X, plan=plan)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, str(case))
    # prefetch distances change no arithmetic: the same bits as one stage ahead
    base = B.Plan.make(kernel=B.KERNEL_TILED, bm=bm, bn=bn, splitk=splitk, wm=4, pf=1, xpf=1)
    assert np.array_equal(C.view(np.uint16), run(p, X, plan=base).view(np.uint16)), case


TILED_K2 = [
    # (M, K, N, bm, bn, splitk, pf): two K slices of four waves; runs of 1,
    # 2, 3, 5 and 86 groups (odd runs leave the second slice's last stage
    # empty), uneven splits, one group per split, ragged rows and columns
    (1, 128, 70, 128, 64, 1, 1),
    (130, 256, 64, 128, 64, 1, 2),
    (200, 384, 100, 128, 64, 1, 2),
    (257, 640, 129, 128, 128, 1, 1),
    (129, 640, 64, 128, 64, 2, 2),
    (300, 1152, 130, 128, 128, 3, 2),
    (128, 1152, 64, 128, 64, 9, 1),
    (150, 11008, 80, 128, 64, 1, 2),
    (260, 11008, 256, 128, 128, 4, 1),
]


@pytest.mark.parametrize("case", TILED_K2, ids=lambda c: "M%d_K%d_N%d_bm%d_bn%d_s%d_pf%d" % c)
def test_tiled_k2_plan(case):
    M, K, N, bm, bn, splitk, pf = case
    log("tiled k2 %s" % (case,))
    p = prob(M, K)
    X = X_for(K, N)
    plan = B.Plan.make(kernel=B.KERNEL_TILED, bm=bm, bn=bn, splitk=splitk, wm=4, wk=2, pf=pf, xpf=1)
    C = run(p, X, plan=plan)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, str(case))


NARROW = [
    # (M, K, N, ncol, pf, splitk, rb, wk[, wm]): 64- or 128-row tiles (48 or
    # 96 with three waves along M) with ragged tails, every column width,
    # columns past N, fewer groups than the ring, remainders of the ring,
    # splits across workgroups and across waves
    (1, 128, 1, 16, 8, 1, 2, 1),
    (100, 384, 9, 16, 8, 1, 1, 1),
    (129, 384, 16, 16, 16, 1, 2, 1),
    (300, 1152, 16, 16, 8, 1, 2, 1),
    (300, 1152, 13, 16, 16, 2, 1, 1),
    (300, 1152, 16, 16, 8, 9, 2, 1),
    (257, 4096, 16, 16, 8, 1, 2, 1),
    (257, 4096, 11, 16, 16, 3, 1, 1),
    (200, 640, 32, 32, 8, 1, 1, 1),
    (200, 640, 17, 32, 16, 2, 2, 1),
    (131, 1152, 31, 32, 8, 3, 2, 1),
    (64, 11008, 32, 32, 8, 5, 1, 1),
    (250, 1152, 64, 64, 8, 1, 2, 1),
    (250, 1152, 33, 64, 16, 2, 1, 1),
    (130, 2048, 64, 64, 8, 4, 2, 1),
    (129, 1152, 3, 64, 16, 1, 1, 1),
    (70, 5120, 20, 32, 16, 3, 1, 1),
    (300, 4096, 16, 16, 8, 1, 1, 2),
    (300, 4096, 16, 16, 8, 1, 1, 4),
    (190, 1152, 9, 16, 8, 2, 2, 4),
    (129, 11008, 24, 32, 8, 6, 1, 2),
    (77, 384, 64, 64, 8, 1, 2, 2),
    (100, 4096, 16, 16, 8, 1, 1, 1, 3),
    (150, 1152, 9, 16, 16, 2, 1, 1, 3),
    (97, 11008, 32, 32, 8, 6, 2, 1, 3),
    (47, 640, 64, 64, 8, 1, 1, 1, 3),
    (300, 4096, 24, 32, 8, 4, 1, 1, 3),
    (300, 4096, 16, 16, 4, 1, 1, 2),
    (190, 1152, 9, 16, 4, 2, 2, 4),
    (70, 640, 5, 16, 4, 1, 1, 1),
    (129, 11008, 32, 32, 4, 6, 2, 2),
]


@pytest.mark.parametrize("case", NARROW, ids=lambda c: "M%d_K%d_N%d_c%d_pf%d_s%d_rb%d_wk%d" % c[:8]
                         + ("_wm%d" % c[8] if len(c) > 8 else ""))
def test_narrow_plan(case):
    M, K, N, ncol, pf, splitk, rb, wk = case[:8]
    wm = case[8] if len(case) > 8 else 4
    log("narrow %s" % (case,))
    p = prob(M, K)
    X = X_for(K, N)
    plan = B.Plan.make(kernel=B.KERNEL_NARROW, ncol=ncol, pf=pf, splitk=splitk, rb=rb, wk=wk, wm=wm)
    C = run(p, X, plan=plan)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, str(case))


@pytest.mark.parametrize("N", [1, 2, 3, 5, 16, 17, 33, 64, 65, 100, 128, 256])
def test_default_dispatch(N):
    M, K = 333, 1152
    log("default N=%d" % N)
    p = prob(M, K)
    X = X_for(K, N, seed=1)
    C = run(p, X)
    C_ref, A_ref = p.reference(X)
    assert_parity(C, C_ref, A_ref, "default N=%d" % N)


def test_gemv_entry_point():
    import torch
    from gpu_util import dev
    M, K = 515, 4096
    p = prob(M, K)
    X = X_for(K, 1, seed=2)
    out = B.gemv(p.qpk, p.s_d, p.zpk, dev(X[:, 0]))
    torch.cuda.synchronize()
    C_ref, A_ref = p.reference(X)
    assert_parity(out.cpu().numpy()[:, None], C_ref, A_ref, "gemv")


def test_repeatable_bitwise():
    """Same plan and inputs give identical bits, split reductions included."""
    M, K = 300, 1152
    p = prob(M, K)
    for N, plan in [(1, None), (16, None), (200, None),
                    (8, B.Plan.make(kernel=1, ncol=8, rb=1, wm=2, wk=2, splitk=3)),
                    (264, B.Plan.make(kernel=2, bm=128, bn=256, splitk=2)),
                    (100, B.Plan.make(kernel=2, bm=128, bn=64, splitk=3, pf=4, xpf=3)),
                    (30, B.Plan.make(kernel=3, ncol=32, pf=8, splitk=3, rb=2, wk=1)),
                    (12, B.Plan.make(kernel=3, ncol=16, pf=8, splitk=1, rb=1, wk=4)),
                    (20, B.Plan.make(kernel=3, ncol=32, pf=8, splitk=4, rb=1, wk=1, wm=3)),
                    (90, B.Plan.make(kernel=2, bm=128, bn=64, wm=4, wk=2, pf=2, splitk=3))]:
        X = X_for(K, N, seed=3)
        a = run(p, X, plan=plan)
        b = run(p, X, plan=plan)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), N
