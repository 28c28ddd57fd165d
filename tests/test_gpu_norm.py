"""Residual add + RMS normalization (alone and as the fused prologue of the
W4A16 product) against the oracle: the stored stream h bit for bit, the
normalized rows within the normalization tolerance, the product within the
GEMM rule computed on the oracle's normalized rows."""

import numpy as np
import pytest
import torch

import oracle.w4a16 as ora
from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import GUARD, Problem, assert_parity, dev, guarded_out, guards_intact, log

pytestmark = pytest.mark.gpu


def norm_ref(x, r, gamma, eps):
    """Stored stream and its normalization (the definition the library
    documents: the mean of squares is taken over the stored fp16 h)."""
    h16 = ora.residual_fp16(x, r)
    y, _ = ora.add_rmsnorm(h16, np.zeros_like(h16), gamma, eps)
    return h16, y


def check_norm(y_gpu, h_gpu, h16, y_ref, what):
    assert np.array_equal(h_gpu.view(np.uint16), h16.view(np.uint16)), what + ": h differs"
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = ora.norm_tolerance(y_ref)
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d bad, max err/tol %.3g" % (what, int(bad.sum()), float(np.max(err / tol)))


NORM_SHAPES = [(1, 4096, 1e-6), (3, 128, 1e-5), (5, 11008, 1e-6), (2, 5120, 0.5), (7, 24576, 1e-6),
               (64, 4096, 1e-6), (1, 8, 1e-6), (33, 1000, 1e-6)]


@pytest.mark.parametrize("case", NORM_SHAPES, ids=lambda c: "N%d_K%d_eps%g" % c)
def test_add_rmsnorm(case):
    N, K, eps = case
    log("add_rmsnorm %s" % (case,))
    x, r, g = inputs.hidden_states(N, K, wid=500 + K)
    h16, y_ref = norm_ref(x, r, g, eps)
    hb, h = guarded_out(N, K)
    yb, y = guarded_out(N, K)
    B.add_rmsnorm(dev(x), dev(r), dev(g), eps, h=h, y=y)
    torch.cuda.synchronize()
    assert guards_intact(hb, N, K) and guards_intact(yb, N, K), "write outside an output"
    check_norm(y.cpu().numpy(), h.cpu().numpy(), h16, y_ref, str(case))


def test_add_rmsnorm_in_place_and_zero_rows():
    """h == residual (in-place update); rows with x = -r normalize to 0."""
    N, K = 6, 4096
    x, r, g = inputs.hidden_states(N, K, wid=510)
    x[2] = -r[2]
    h16, y_ref = norm_ref(x, r, g, 1e-6)
    rd = dev(r)
    y, h = B.add_rmsnorm(dev(x), rd, dev(g), 1e-6, h=rd)
    torch.cuda.synchronize()
    assert h.data_ptr() == rd.data_ptr()
    check_norm(y.cpu().numpy(), rd.cpu().numpy(), h16, y_ref, "in place")
    assert np.all(y.cpu().numpy()[2] == 0)


_probs = {}


def prob(M, K):
    if (M, K) not in _probs:
        _probs[(M, K)] = Problem(M, K, seed=60 + len(_probs))
    return _probs[(M, K)]


def run_fused(p, N, plan=None, eps=1e-6, wid=520, in_place=False):
    M, K = p.M, p.K
    x, r, g = inputs.hidden_states(N, K, wid=wid)
    h16, y_ref = norm_ref(x, r, g, eps)
    cb, c = guarded_out(N, M)
    rd = dev(r)
    hb, h = (None, rd) if in_place else guarded_out(N, K)
    B.gemm_add_rmsnorm(p.qpk, p.s_d, p.zpk, dev(x), rd, dev(g), eps, h=h, out=c, plan=plan)
    torch.cuda.synchronize()
    assert guards_intact(cb, N, M), "write outside c"
    if hb is not None:
        assert guards_intact(hb, N, K), "write outside h"
    assert np.array_equal(h.cpu().numpy().view(np.uint16), h16.view(np.uint16)), "h differs"
    return np.ascontiguousarray(c.cpu().numpy().T), y_ref


FUSED = [
    # (M, K, N, plan fields or None for the default)
    (300, 1152, 1, None),
    (77, 1152, 3, None),
    (96, 1152, 8, dict(kernel=1, ncol=8, rb=1, wm=2, wk=2, splitk=3)),
    (130, 4096, 1, dict(kernel=1, ncol=1, rb=1, wm=1, wk=8, splitk=2)),
    (300, 1152, 16, None),
    (257, 4096, 11, dict(kernel=3, ncol=16, pf=16, splitk=3, rb=1, wk=1)),
    (131, 1152, 31, dict(kernel=3, ncol=32, pf=8, splitk=3, rb=2, wk=1)),
    (300, 4096, 16, dict(kernel=3, ncol=16, pf=8, splitk=1, rb=1, wk=4)),
    (333, 1152, 100, None),
    (257, 1152, 264, dict(kernel=2, bm=128, bn=256, splitk=2, wm=2)),
    (129, 384, 130, dict(kernel=2, bm=256, bn=128, splitk=2, wm=4)),
    (64, 11008, 5, None),
    # the one-launch prologue inside the skinny kernel: waves along M and K
    (200, 1152, 4, dict(kernel=1, ncol=4, rb=1, wm=2, wk=4, splitk=1)),
    (77, 1152, 8, dict(kernel=1, ncol=8, rb=1, wm=2, wk=2, splitk=1)),
    (33, 4096, 2, dict(kernel=1, ncol=2, rb=1, wm=1, wk=16, splitk=1)),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "M%d_K%d_N%d_%s" % (c[0], c[1], c[2],
                                                                          "default" if c[3] is None else
                                                                          "k%d" % c[3]["kernel"]))
def test_gemm_add_rmsnorm(case):
    M, K, N, fields = case
    log("gemm_add_rmsnorm %s" % (case,))
    p = prob(M, K)
    plan = None if fields is None else B.Plan.make(**fields)
    C, y_ref = run_fused(p, N, plan=plan)
    C_ref, A_ref = ora.reference(p.qpk_ref, p.s, p.zpk_ref, y_ref.T)
    assert_parity(C, C_ref, A_ref, str(case))


def test_gemm_add_rmsnorm_in_place():
    p = prob(300, 1152)
    for N in (1, 16, 100):
        C, y_ref = run_fused(p, N, wid=530, in_place=True)
        C_ref, A_ref = ora.reference(p.qpk_ref, p.s, p.zpk_ref, y_ref.T)
        assert_parity(C, C_ref, A_ref, "in place N=%d" % N)


@pytest.mark.parametrize("case", [(-20, 1, 1, 8), (-12, 1, 2, 8), (-12, 4, 2, 8), (10, 1, 1, 8), (10, 3, 2, 4),
                                  (0, 2, 1, 16)],
                         ids=lambda c: "scale2^%d_N%d_wm%d_wk%d" % c)
def test_gemm_add_rmsnorm_scaled_stream(case):
    """The one-launch prologue stages fp16(h gamma 2^e), e a power of two per
    wave and token: a residual stream of small (2^-12) or large (2^10)
    magnitude (2^-20: fp16 subnormal inputs) still meets the GEMM rule on
    the oracle's normalized rows.
    eps = 0, where the normalization is scale-invariant; the skinny plan of
    one split (the one-launch form) forced, with waves along M and K."""
    ex, N, wm, wk = case
    M, K = 300, 4096
    log("gemm_add_rmsnorm scaled %s" % (case,))
    p = prob(M, K)
    x, r, g = inputs.hidden_states(N, K, wid=550 + N)
    x = (x.astype(np.float64) * 2.0 ** ex).astype(np.float16)
    r = (r.astype(np.float64) * 2.0 ** ex).astype(np.float16)
    h16, y_ref = norm_ref(x, r, g, 0.0)
    plan = B.Plan.make(kernel=1, ncol=N, rb=1, wm=wm, wk=wk, splitk=1)
    cb, c = guarded_out(N, M)
    hb, h = guarded_out(N, K)
    B.gemm_add_rmsnorm(p.qpk, p.s_d, p.zpk, dev(x), dev(r), dev(g), 0.0, h=h, out=c, plan=plan)
    torch.cuda.synchronize()
    assert guards_intact(cb, N, M) and guards_intact(hb, N, K), "write outside an output"
    assert np.array_equal(h.cpu().numpy().view(np.uint16), h16.view(np.uint16)), "h differs"
    C = np.ascontiguousarray(c.cpu().numpy().T)
    C_ref, A_ref = ora.reference(p.qpk_ref, p.s, p.zpk_ref, y_ref.T)
    assert_parity(C, C_ref, A_ref, str(case))


@pytest.mark.parametrize("shape", [(12288, 4096, 1), (12288, 4096, 16), (22016, 4096, 1), (22016, 4096, 128)],
                         ids=lambda s: "M%d_K%d_N%d" % s)
def test_gemm_add_rmsnorm_full_size(shape):
    """The QKV and gate/up projections of LLaMA-7B with their prologue, at
    decode and prefill widths, on sampled rows."""
    M, K, N = shape
    log("gemm_add_rmsnorm full %s" % (shape,))
    p = prob(M, K)
    C, y_ref = run_fused(p, N, wid=540)
    rows = np.random.default_rng(M + N).choice(M, 64, replace=False)
    C_ref, A_ref = ora.reference_rows(p.qpk_ref, p.s, p.zpk_ref, y_ref.T, rows)
    assert_parity(C[rows], C_ref, A_ref, "full %s" % (shape,))
