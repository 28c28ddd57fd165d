"""Helpers of the GPU parity tests: seeded inputs, device packing through the
C ABI, oracle comparison, output poisoning and guard checks."""

import sys

import numpy as np
import torch

import oracle.w4a16 as ora
from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs

GUARD = 64          # fp16 guard elements on each side of an output buffer
POISON = 0x7E00     # fp16 quiet NaN bit pattern
GUARD_BITS = 0x5A5A


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Problem:
    """One weight matrix on host and device (packed on the device)."""

    def __init__(self, M, K, seed=0, q=None, s=None, z=None, check_pack=True):
        if q is None:
            q, s, z = inputs.weights(M, K, wid=100 + seed, layer=M, proj=K)
        self.M, self.K = M, K
        self.q, self.s, self.z = q, s, z
        self.qpk_ref, self.zpk_ref = ora.pack(q, z)
        qd, zd = dev(q), dev(z)
        qpk, zpk = B.pack(qd, zd)
        torch.cuda.synchronize()
        self.qpk, self.zpk = qpk, zpk
        self.s_d = dev(s)
        if check_pack:
            got_q = qpk.cpu().numpy().view(np.uint32)
            got_z = zpk.cpu().numpy().view(np.uint32)
            assert np.array_equal(got_q, self.qpk_ref), "packed weights differ"
            assert np.array_equal(got_z, self.zpk_ref), "packed zeros differ"

    def reference(self, X):
        return ora.reference(self.qpk_ref, self.s, self.zpk_ref, X)

    def reference_rows(self, X, rows):
        return ora.reference_rows(self.qpk_ref, self.s, self.zpk_ref, X, rows)


def guarded_out(M, N):
    """An output [M, N] view inside a buffer with guard elements on both
    sides; the view is poisoned with NaN, the guards hold a fixed pattern."""
    total = M * N + 2 * GUARD
    buf = torch.full((total,), GUARD_BITS, dtype=torch.int16, device="cuda")
    buf[GUARD:GUARD + M * N] = POISON
    out = buf[GUARD:GUARD + M * N].view(torch.float16).view(M, N)
    return buf, out


def guards_intact(buf, M, N):
    h = buf.cpu().numpy().view(np.uint16)
    return bool(np.all(h[:GUARD] == GUARD_BITS) and np.all(h[GUARD + M * N:] == GUARD_BITS))


def run(prob, X, plan=None, guard=True, layout=B.LAYOUT_KN):
    """Run the GEMM on the GPU; returns the fp16 result as numpy [M, N].
    X is always given as [K, N]; with the token layout it goes to the device
    as [N, K] and the [N, M] result comes back transposed."""
    M, N = prob.M, X.shape[1]
    token = layout == B.LAYOUT_TOKEN
    xd = dev(X.T if token else X)
    shape = (N, M) if token else (M, N)
    if guard:
        buf, out = guarded_out(*shape)
    else:
        buf, out = None, torch.empty(shape, dtype=torch.float16, device="cuda")
    B.gemm(prob.qpk, prob.s_d, prob.zpk, xd, out=out, plan=plan, layout=layout)
    torch.cuda.synchronize()
    if guard:
        assert guards_intact(buf, M, N), "write outside the output"
    res = out.cpu().numpy()
    return np.ascontiguousarray(res.T) if token else res


def assert_parity(C_gpu, C_ref, A_ref, what=""):
    r = ora.check(C_gpu, C_ref, A_ref)
    assert r["ok"], "%s: %d bad (%d non-finite), max err/tol %.3g, max |err| %.3g" % (
        what, r["n_bad"], r["n_nonfinite"], r["max_err_over_tol"], r["max_abs_err"])
    return r
