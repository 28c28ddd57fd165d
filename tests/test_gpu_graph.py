"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed several times, with eager work and synchronisations between the
replays: every replay equals the eager result bit for bit.  Covers the
split reductions (arrival counters left at zero for the next replay), the
activation rewrites and the decode attention's split merge."""

import numpy as np
import pytest
import torch

from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import Problem, dev, log

pytestmark = pytest.mark.gpu

CALLS = [
    # (M, K, N, layout, plan fields)
    (300, 1152, 1, B.LAYOUT_KN, dict(kernel=1, ncol=1, rb=1, wm=2, wk=2, splitk=3)),
    (300, 1152, 6, B.LAYOUT_TOKEN, dict(kernel=1, ncol=6, rb=1, wm=1, wk=2, splitk=2)),
    (257, 4096, 11, B.LAYOUT_KN, dict(kernel=3, ncol=16, pf=16, splitk=3, rb=1, wk=1)),
    (257, 1152, 264, B.LAYOUT_TOKEN, dict(kernel=2, bm=128, bn=256, splitk=2, wm=2)),
]


@pytest.mark.parametrize("case", CALLS, ids=lambda c: "M%d_N%d_k%d" % (c[0], c[2], c[4]["kernel"]))
def test_gemm_graph_replays(case):
    M, K, N, layout, fields = case
    log("graph gemm %s" % (case[:3],))
    p = Problem(M, K, seed=400 + N)
    X = inputs.activations(K, N, wid=900 + N)
    xd = dev(X.T if layout == B.LAYOUT_TOKEN else X)
    plan = B.Plan.make(**fields)
    ws = B.Workspace()
    eager = B.gemm(p.qpk, p.s_d, p.zpk, xd, plan=plan, layout=layout, workspace=ws).clone()
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        B.gemm(p.qpk, p.s_d, p.zpk, xd, out=out, plan=plan, layout=layout, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        B.gemm(p.qpk, p.s_d, p.zpk, xd, out=out, plan=plan, layout=layout, workspace=ws)
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(4096, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay %d" % r


def test_attention_graph_replays():
    """The split attention writes the cache at the position, so each replay
    runs on a fresh copy of the caches; outputs and caches match eager."""
    Bn, H, D, S = 2, 8, 128, 2048
    qkv, kc, vc = inputs.attention_inputs(Bn, H, D, S, wid=950)
    pos = dev(np.array([2047, 1000], dtype=np.int32))
    qd = dev(qkv)
    ke, ve = dev(kc), dev(vc)
    ws = B.Workspace()
    eager = B.decode_attention(qd, ke, ve, pos, workspace=ws).clone()
    kg, vg = dev(kc), dev(vc)
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        B.decode_attention(qd, kg, vg, pos, out=out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        B.decode_attention(qd, kg, vg, pos, out=out, workspace=ws)
    for r in range(3):
        kg.copy_(dev(kc))
        vg.copy_(dev(vc))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay %d" % r
        assert torch.equal(kg.view(torch.int16), ke.view(torch.int16)), "replay %d" % r
        assert torch.equal(vg.view(torch.int16), ve.view(torch.int16)), "replay %d" % r
