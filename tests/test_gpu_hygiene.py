"""Input validation through the binding on a real device, and the pack
kernel's bit-exactness against the oracle for every row length class."""

import numpy as np
import pytest
import torch

import oracle.w4a16 as ora
from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import dev, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K", [(1, 128), (3, 4096), (64, 11008), (17, 384), (5, 1024)])
def test_pack_bit_exact(M, K):
    log("pack %dx%d" % (M, K))
    q = inputs.uniform_codes((M, K), seed=M * K)
    z = inputs.uniform_codes((M, K // 128), seed=M + K)
    # codes above 15 must contribute their low nibble only
    q[0, :3] = [0x1F, 0xF0, 0xAB]
    qpk, zpk = B.pack(dev(q), dev(z))
    qz, _ = B.pack(dev(q), None)
    _, zz = B.pack(None, dev(z))
    torch.cuda.synchronize()
    want_q, want_z = ora.pack(q, z)
    for got, want in ((qpk, want_q), (zpk, want_z), (qz, want_q), (zz, want_z)):
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want)


def test_binding_rejects_bad_tensors():
    M, K = 16, 256
    q = dev(inputs.uniform_codes((M, K), 1))
    z = dev(inputs.uniform_codes((M, 2), 2))
    qpk, zpk = B.pack(q, z)
    s = torch.ones((M, 2), dtype=torch.float16, device="cuda")
    x = torch.ones((K, 4), dtype=torch.float16, device="cuda")
    with pytest.raises(TypeError):
        B.gemm(qpk, s.float(), zpk, x)
    with pytest.raises(ValueError):
        B.gemm(qpk, s, zpk, torch.ones((K + 8, 4), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        B.gemm(qpk, s, zpk, x.t())            # not contiguous
    with pytest.raises(B.W4A16Error) as e:
        B.gemm(qpk, s, zpk, x, plan=B.Plan.make(kernel=2, bm=64, bn=64, splitk=1))
    assert e.value.status == 2
    # an output view 2 bytes past an aligned base: rejected as misaligned
    out = torch.empty((M * 4 + 1,), dtype=torch.float16, device="cuda")[1:].view(M, 4)
    with pytest.raises(B.W4A16Error) as e:
        B.gemm(qpk, s, zpk, x, out=out)
    assert e.value.status == 3
