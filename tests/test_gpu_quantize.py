"""The round-to-nearest group quantizer on the GPU against the oracle's
quantizer (oracle.quantize_rtn, then oracle.pack): packed codes, fp16
scales and packed zeros bit for bit, on random weights with outliers and on
the degenerate groups the min/max form has (all zero, constant, one sign,
a single nonzero, extreme magnitudes, zero-word padding); then the
quantized matrix through the GEMM against the oracle product."""

import numpy as np
import pytest
import torch

import oracle.w4a16 as ora
from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import assert_parity, dev, log

pytestmark = pytest.mark.gpu


def quantize_both(W):
    wd = dev(W)
    qpk, s, zpk = B.quantize(wd)
    torch.cuda.synchronize()
    q_ref, s_ref, z_ref = ora.quantize_rtn(W)
    qpk_ref, zpk_ref = ora.pack(q_ref, z_ref)
    return (qpk.cpu().numpy().view(np.uint32), s.cpu().numpy(), zpk.cpu().numpy().view(np.uint32),
            qpk_ref, s_ref, zpk_ref)


def assert_same(W, what):
    g_q, g_s, g_z, r_q, r_s, r_z = quantize_both(W)
    assert np.array_equal(g_s.view(np.uint16), r_s.view(np.uint16)), "%s: scales differ" % what
    assert np.array_equal(g_z, r_z), "%s: zeros differ" % what
    bad = np.argwhere(g_q != r_q)
    assert bad.size == 0, "%s: packed codes differ at %s" % (what, bad[:5].tolist())


@pytest.mark.parametrize("M,K", [(1, 128), (17, 384), (64, 11008), (300, 4096), (33, 1152)])
def test_random_weights(M, K):
    log("quantize %dx%d" % (M, K))
    W = inputs.fp16_weights(M, K, wid=300, layer=M, proj=K)
    assert_same(W, "random %dx%d" % (M, K))


def test_degenerate_groups():
    M, K = 8, 1024
    W = inputs.fp16_weights(M, K, wid=301).astype(np.float32)
    g = lambda r, j: (r, slice(128 * j, 128 * (j + 1)))
    W[g(0, 0)] = 0.0                      # all zero: s from the 1e-5 floor, z = 0
    W[g(0, 1)] = 0.25                     # constant positive: lo = 0
    W[g(0, 2)] = -0.25                    # constant negative: hi = 0, z = 15
    W[g(1, 0)] = np.abs(W[g(1, 0)])       # one sign
    W[g(1, 1)] = -np.abs(W[g(1, 1)])
    W[g(2, 0)] = 0.0
    W[2, 5] = 0.5                         # a single nonzero
    W[g(3, 0)] = np.linspace(-60000, 60000, 128)   # extreme magnitudes
    W[g(3, 1)] = np.linspace(-1e-4, 1e-4, 128)     # tiny range: fp16 subnormal scale
    W[4] = np.tile(np.arange(16, dtype=np.float32) * 0.01, K // 16)   # exact grid
    W = W.astype(np.float16)
    assert_same(W, "degenerate")


def test_quantize_then_gemm():
    M, K, N = 257, 2048, 9
    W = inputs.fp16_weights(M, K, wid=302)
    qpk, s, zpk = B.quantize(dev(W))
    X = inputs.activations(K, N, wid=302)
    out = B.gemm(qpk, s, zpk, dev(X))
    torch.cuda.synchronize()
    q_ref, s_ref, z_ref = ora.quantize_rtn(W)
    qpk_ref, zpk_ref = ora.pack(q_ref, z_ref)
    C_ref, A_ref = ora.reference(qpk_ref, s_ref, zpk_ref, X)
    assert_parity(out.cpu().numpy(), C_ref, A_ref, "quantize then gemm")
