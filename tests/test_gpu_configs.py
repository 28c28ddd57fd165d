"""Parity at the full workload sizes, with the default dispatch that the
bench times: the 4096x4096 GEMV, the four LLaMA-7B decode linears, the
12288x4096 small-N and large-N sweeps, and the 32-layer stack at N = 1 and
N = 16.  Every element is compared where the CPU oracle finishes in seconds;
the largest products are compared on sampled rows (boundary rows of every
tile size plus random rows), which the oracle computes one by one."""

import numpy as np
import pytest
import torch

import oracle.w4a16 as ora
from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import Problem, assert_parity, dev, log, run

pytestmark = pytest.mark.gpu


def sample_rows(M, seed, n_random=96):
    # first and last rows of 16-, 32-, 64-, 128-, 256- and 512-row tiles
    rows = set([0, 1, 15, 16, 17, 31, 32, 63, 64, 127, 128, 255, 256, 383, 384, 511, 512, 513,
                767, 768, 1023, 1024, 1025, 1535, 1536, M - 1, M - 2, M - 17, M - 256, M - 512, M - 513])
    rng = np.random.default_rng(seed)
    rows.update(int(r) for r in rng.integers(0, M, n_random))
    return np.array(sorted(r for r in rows if 0 <= r < M))


def full_problem(wid, M, K, proj=0, layer=0):
    q, s, z = inputs.weights(M, K, wid=wid, layer=layer, proj=proj)
    return Problem(M, K, q=q, s=s, z=z)


def test_gemv_4096x4096():
    p = full_problem(1, 4096, 4096)
    X = inputs.activations(4096, 1, wid=1)
    log("gemv 4096x4096")
    C = run(p, X)
    C_ref, A_ref = p.reference(X)
    r = assert_parity(C, C_ref, A_ref, "gemv_4096x4096")
    log("  max err/tol %.3g, max |err|/A %.3g" % (r["max_err_over_tol"], r["max_rel_to_A"]))


@pytest.mark.parametrize("proj", range(4), ids=[p[0] for p in inputs.LLAMA7B_PROJ])
def test_llama7b_decode_linear(proj):
    name, M, K = inputs.LLAMA7B_PROJ[proj]
    p = full_problem(2, M, K, proj=proj)
    X = inputs.activations(K, 1, wid=2, proj=proj)
    log("decode %s %dx%d" % (name, M, K))
    C = run(p, X)
    C_ref, A_ref = p.reference(X)
    r = assert_parity(C, C_ref, A_ref, name)
    log("  max err/tol %.3g, max |err|/A %.3g" % (r["max_err_over_tol"], r["max_rel_to_A"]))


@pytest.fixture(scope="module")
def w12288():
    return full_problem(3, 12288, 4096)


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 32])
def test_small_n_12288x4096(w12288, N):
    X = inputs.activations(4096, N, wid=3)
    log("small-N 12288x4096 N=%d" % N)
    C = run(w12288, X)
    C_ref, A_ref = w12288.reference(X)
    assert_parity(C, C_ref, A_ref, "small N=%d" % N)


@pytest.fixture(scope="module")
def w12288b():
    return full_problem(4, 12288, 4096)


@pytest.mark.parametrize("N", [64, 128, 256, 512, 1024, 2048, 4096])
def test_large_n_12288x4096(w12288b, N):
    X = inputs.activations(4096, N, wid=4)
    log("large-N 12288x4096 N=%d" % N)
    C = run(w12288b, X, guard=N <= 1024)
    if N <= 512:
        C_ref, A_ref = w12288b.reference(X)
        assert_parity(C, C_ref, A_ref, "large N=%d" % N)
    else:
        rows = sample_rows(12288, N)
        C_ref, A_ref = w12288b.reference_rows(X, rows)
        assert_parity(C[rows], C_ref, A_ref, "large N=%d (rows)" % N)
        assert np.all(np.isfinite(C)), "non-finite output"


@pytest.mark.parametrize("N", [1, 16])
def test_llama7b_stack(N):
    """32 layers x 4 linears back to back (one decode step), packed weight
    words drawn directly, activations re-seeded per layer; every call is
    checked on sampled rows and for finiteness."""
    L = 32
    mats = []
    for layer in range(L):
        for proj, (name, M, K) in enumerate(inputs.LLAMA7B_PROJ):
            words = inputs.raw_q_words(M, K, wid=5, layer=layer, proj=proj)
            s, z = inputs.scales_zeros(M, K, wid=5, layer=layer, proj=proj)
            rows = sample_rows(M, 1000 * layer + proj, n_random=24)
            zpk_ref = ora.pack_nibbles(z)
            qd = dev(words.view(np.int32))
            _, zd = B.pack(None, dev(z))
            if layer == 0:
                torch.cuda.synchronize()
                assert np.array_equal(zd.cpu().numpy().view(np.uint32), zpk_ref)
            mats.append(dict(name=name, M=M, K=K, qd=qd, zd=zd, sd=dev(s), rows=rows,
                             words=words[rows].copy(), s=s[rows].copy(), zpk=zpk_ref[rows].copy(),
                             X=inputs.activations(K, N, wid=5, layer=layer, proj=proj)))
            del words
    log("stack N=%d: %d matrices resident" % (N, len(mats)))
    outs = []
    xs = [dev(m["X"]) for m in mats]
    for m, xd in zip(mats, xs):
        outs.append(B.gemm(m["qd"], m["sd"], m["zd"], xd))
    torch.cuda.synchronize()
    for m, o in zip(mats, outs):
        C = o.cpu().numpy()
        assert np.all(np.isfinite(C)), m["name"]
        C_ref, A_ref = ora.reference(m["words"], m["s"], m["zpk"], m["X"])
        assert_parity(C[m["rows"]], C_ref, A_ref, "stack %s" % m["name"])
