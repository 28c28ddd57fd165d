"""w4a16_gemm_noalloc (the entry point for callers that cannot allocate)
against w4a16_gemm: the same default plan and kernels, so the results must
agree bit for bit, and both must pass the oracle's rule.  Two calls in a
row share the library's device scratch, the second with a smaller input;
a shape whose scratch need exceeds the fixed maximum is refused and writes
nothing."""

import numpy as np
import pytest
import torch

from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import GUARD, Problem, assert_parity, dev, guarded_out, guards_intact, log

pytestmark = pytest.mark.gpu

# (M, K, N) pairs: the first call, then a smaller one (split-K narrow,
# tiled reading x in place and through activation chunks (N not a multiple
# of 8), skinny with and without a workspace)
PAIRS = [
    ((12288, 4096, 32), (4096, 4096, 16)),
    ((12288, 4096, 64), (4096, 11008, 8)),
    ((12288, 4096, 128), (1000, 4096, 40)),
    ((12288, 4096, 100), (4096, 4096, 60)),
    ((12288, 4096, 1), (200, 1152, 1)),
    ((22016, 4096, 4), (4096, 11008, 2)),
]


def _one(M, K, N, seed):
    p = Problem(M, K, seed=seed)
    X = inputs.activations(K, N, wid=20 + seed)
    xd = dev(X)
    want = B.gemm(p.qpk, p.s_d, p.zpk, xd)            # w4a16_gemm, binding-provided workspace
    buf, out = guarded_out(M, N)
    B.gemm_noalloc(p.qpk, p.s_d, p.zpk, xd, out)       # w4a16_gemm_noalloc
    torch.cuda.synchronize()
    assert guards_intact(buf, M, N), "write outside the output"
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.cpu().numpy().view(np.uint16)), (M, K, N)
    C_ref, A_ref = p.reference(X)
    assert_parity(got, C_ref, A_ref, "noalloc %dx%d N=%d" % (M, K, N))


@pytest.mark.parametrize("first,second", PAIRS, ids=["%dx%dn%d_then_%dx%dn%d" % (a + b) for a, b in PAIRS])
def test_noalloc_matches_gemm_twice(first, second):
    log("noalloc %s then %s (plans %s / %s)" % (first, second, B.plan_default(first[0], first[2], first[1]).as_dict(),
                                                B.plan_default(second[0], second[2], second[1]).as_dict()))
    _one(*first, seed=1)
    _one(*second, seed=2)


def test_noalloc_refuses_oversize():
    # N not a multiple of 8: the tiled plan needs the 2 K N bytes of
    # activation chunks, above the scratch
    M, K, N = 12288, 4096, 4095
    need = B.workspace_size(M, N, K)
    cap = int(B.lib().w4a16_gemm_noalloc_max_bytes())
    assert cap == 16 << 20 and need > cap
    log("noalloc refusal: need %d > %d" % (need, cap))
    p = Problem(M, K, seed=3, check_pack=False)
    x = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    buf, out = guarded_out(M, N)
    st = B.lib().w4a16_gemm_noalloc(p.qpk.data_ptr(), p.s_d.data_ptr(), p.zpk.data_ptr(), x.data_ptr(),
                                    out.data_ptr(), M, N, K, 128, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 4, st   # W4A16_ERR_WORKSPACE
    assert b"scratch" in B.lib().w4a16_last_error()
    h = buf.cpu().numpy().view(np.uint16)
    assert np.all(h[GUARD:GUARD + M * N] == 0x7E00), "a refused call wrote its output"
