"""Exact structural gates on the GPU, for every kernel, every default plan of
the measured workloads and the fused prologues.

The format of the PerfXLLM page on Snapdragon 8 Gen2 (§3.1: one scale and
one zero per group of 128 weights) has three consequences that hold exactly,
whatever the accumulation order:

* q == z gives C = 0 (|C| <= 1e-3 on the device: the tolerance with A = 0);
* an identity activation column e_k gives the dequantized weight column
  Wdeq[:, k], rounded once to fp16 (bit for bit; chosen k sit on octet,
  group and tail boundaries, K = 11008 included for its 86-group tail);
* q = 15, z = 0, s = fp16(0.02), X = 1, K = 4096 gives 4096 * 15 * s =
  1229.0625 exactly, 1229.0 in fp16.

Random inputs under the loose tolerance can hide a dropped or shifted
group; these cannot.  The default plans are those the library picks at the
full workload sizes (4096x4096; the LLaMA-7B decode linears at N = 1 and
N = 16; 12288x4096 across the small-N and large-N sweeps), each run here on
a few tiles of rows with a ragged last tile."""

import numpy as np
import pytest
import torch

from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import Problem, dev, log, run

pytestmark = pytest.mark.gpu

SK, TI, NA = B.KERNEL_SKINNY, B.KERNEL_TILED, B.KERNEL_NARROW
KN, TOK = B.LAYOUT_KN, B.LAYOUT_TOKEN


# ---- the default plans of the measured workloads: (M, K, N, layout); each
# is resolved inside the test (the plan choice is the library's)
WORKLOADS = [(4096, 4096, 1, KN)]
WORKLOADS += [(M, K, N, KN) for N in (1, 16) for (_, M, K) in inputs.LLAMA7B_PROJ if (M, K) != (4096, 4096) or N == 16]
WORKLOADS += [(12288, 4096, N, KN) for N in (2, 4, 8, 32, 64, 128, 256, 512, 1024, 2048, 4096)]
WORKLOADS += [(12288, 4096, N, TOK) for N in (1, 8, 16, 64, 4096)]


def _default_cases():
    return [("default_%dx%d_n%d%s" % (M, K, N, "_tok" if layout == TOK else ""), ("default", M), K, N, layout)
            for (M, K, N, layout) in WORKLOADS]


def _resolve(spec, K, N, layout):
    if isinstance(spec, tuple) and spec[0] == "default":
        return B.plan_default(spec[1], N, K, layout)
    return spec


def _mk(**kw):
    return B.Plan.make(**kw)


# ---- explicit plans: every narrow and tiled variant the tuner may pick,
# activations read in place (N a multiple of 8, [K, N]) and re-laid
EXPLICIT = [
    ("narrow_c16_rb1_wk1_dx", _mk(kernel=NA, ncol=16, pf=8, rb=1, wk=1, splitk=1), 4096, 16, KN),
    ("narrow_c16_pf16_rb2_relaid", _mk(kernel=NA, ncol=16, pf=16, rb=2, wk=1, splitk=1), 4096, 13, KN),
    ("narrow_c16_wk2_split2", _mk(kernel=NA, ncol=16, pf=8, rb=2, wk=2, splitk=2), 4096, 16, KN),
    ("narrow_c16_wk4_n8", _mk(kernel=NA, ncol=16, pf=8, rb=1, wk=4, splitk=1), 4096, 8, KN),
    ("narrow_c16_token", _mk(kernel=NA, ncol=16, pf=8, rb=1, wk=2, splitk=2), 4096, 16, TOK),
    ("narrow_c32_wk2_split2", _mk(kernel=NA, ncol=32, pf=8, rb=1, wk=2, splitk=2), 4096, 32, KN),
    ("narrow_c32_pf16_rb2_relaid", _mk(kernel=NA, ncol=32, pf=16, rb=2, wk=1, splitk=2), 4096, 27, KN),
    ("narrow_c32_wk4_split4", _mk(kernel=NA, ncol=32, pf=8, rb=1, wk=4, splitk=4), 4096, 24, KN),
    ("narrow_c64_split4_dx", _mk(kernel=NA, ncol=64, pf=8, rb=1, wk=1, splitk=4), 4096, 64, KN),
    ("narrow_c64_rb2_wk2_relaid", _mk(kernel=NA, ncol=64, pf=8, rb=2, wk=2, splitk=4), 4096, 50, KN),
    ("narrow_c64_pf16_wk4_split8", _mk(kernel=NA, ncol=64, pf=16, rb=1, wk=4, splitk=8), 4096, 40, KN),
    ("narrow_c16_k11008", _mk(kernel=NA, ncol=16, pf=8, rb=1, wk=2, splitk=3), 11008, 16, KN),
    ("narrow_c16_wm3_dx", _mk(kernel=NA, ncol=16, pf=8, rb=1, wk=1, wm=3, splitk=1), 4096, 16, KN),
    ("narrow_c16_wm3_n8", _mk(kernel=NA, ncol=16, pf=8, rb=1, wk=1, wm=3, splitk=1), 4096, 8, KN),
    ("narrow_c32_wm3_rb2_split6", _mk(kernel=NA, ncol=32, pf=8, rb=2, wk=1, wm=3, splitk=6), 11008, 32, KN),
    ("narrow_c16_wm3_pf16_token", _mk(kernel=NA, ncol=16, pf=16, rb=1, wk=1, wm=3, splitk=2), 4096, 16, TOK),
    ("tiled_512x128_w8_pf2", _mk(kernel=TI, bm=512, bn=128, wm=8, pf=2, splitk=1), 4096, 136, KN),
    ("tiled_512x128_w8_split2", _mk(kernel=TI, bm=512, bn=128, wm=8, pf=2, splitk=2), 4096, 100, KN),
    ("tiled_128x128_w4", _mk(kernel=TI, bm=128, bn=128, wm=4, pf=1, splitk=1), 4096, 136, KN),
    ("tiled_128x128_w4_pf2", _mk(kernel=TI, bm=128, bn=128, wm=4, pf=2, splitk=1), 4096, 136, KN),
    ("tiled_256x128", _mk(kernel=TI, bm=256, bn=128, wm=4, pf=1, splitk=1), 4096, 264, KN),
    ("tiled_256x256_2x2", _mk(kernel=TI, bm=256, bn=256, wm=2, pf=1, splitk=1), 4096, 300, KN),
    ("tiled_128x256_2x2", _mk(kernel=TI, bm=128, bn=256, wm=2, pf=1, splitk=1), 4096, 200, KN),
    ("tiled_128x64_split2", _mk(kernel=TI, bm=128, bn=64, wm=4, pf=1, splitk=2), 4096, 70, KN),
    ("tiled_256x64_pf2_split4", _mk(kernel=TI, bm=256, bn=64, wm=4, pf=2, splitk=4), 4096, 64, KN),
    ("tiled_512x128_k11008", _mk(kernel=TI, bm=512, bn=128, wm=8, pf=2, splitk=1), 11008, 24, KN),
    ("tiled_128x64_token", _mk(kernel=TI, bm=128, bn=64, wm=4, pf=1, splitk=1), 4096, 40, TOK),
    ("tiled_128x64_p42_split3", _mk(kernel=TI, bm=128, bn=64, wm=4, pf=4, xpf=2, splitk=3), 4096, 64, KN),
    ("tiled_128x64_p43_split4", _mk(kernel=TI, bm=128, bn=64, wm=4, pf=4, xpf=3, splitk=4), 4096, 100, KN),
    ("tiled_128x128_p32_split2", _mk(kernel=TI, bm=128, bn=128, wm=4, pf=3, xpf=2, splitk=2), 4096, 136, KN),
    ("tiled_256x64_p22_split3", _mk(kernel=TI, bm=256, bn=64, wm=4, pf=2, xpf=2, splitk=3), 4096, 72, KN),
    ("tiled_128x64_p43_k11008", _mk(kernel=TI, bm=128, bn=64, wm=4, pf=4, xpf=3, splitk=3), 11008, 64, KN),
    ("tiled_128x64_p42_token", _mk(kernel=TI, bm=128, bn=64, wm=4, pf=4, xpf=2, splitk=2), 4096, 64, TOK),
    ("tiled_96x64_w3_pf2_split2", _mk(kernel=TI, bm=96, bn=64, wm=3, pf=2, splitk=2), 4096, 64, KN),
    ("tiled_96x64_w3_pf1_k11008", _mk(kernel=TI, bm=96, bn=64, wm=3, pf=1, splitk=3), 11008, 48, KN),
    ("tiled_96x64_w3_token", _mk(kernel=TI, bm=96, bn=64, wm=3, pf=2, splitk=1), 4096, 72, TOK),
    ("tiled_k2_128x64_split2", _mk(kernel=TI, bm=128, bn=64, wm=4, wk=2, pf=2, splitk=2), 4096, 64, KN),
    ("tiled_k2_128x64_odd_k11008", _mk(kernel=TI, bm=128, bn=64, wm=4, wk=2, pf=2, splitk=1), 11008, 100, KN),
    ("tiled_k2_128x128_split3", _mk(kernel=TI, bm=128, bn=128, wm=4, wk=2, pf=1, splitk=3), 4096, 136, KN),
    ("tiled_k2_128x128_token", _mk(kernel=TI, bm=128, bn=128, wm=4, wk=2, pf=2, splitk=1), 4096, 200, TOK),
    ("skinny_c1_wk4", _mk(kernel=SK, ncol=1, rb=1, wm=1, wk=4, splitk=1), 4096, 1, KN),
    ("skinny_c16_split", _mk(kernel=SK, ncol=16, rb=1, wm=2, wk=4, splitk=4), 4096, 16, KN),
    ("skinny_c32_split8", _mk(kernel=SK, ncol=32, rb=1, wm=1, wk=2, splitk=8), 4096, 32, KN),
    ("skinny_c5_token", _mk(kernel=SK, ncol=5, rb=1, wm=2, wk=2, splitk=2), 4096, 5, TOK),
]

CASES = _default_cases() + EXPLICIT


def _rows(plan):
    """Two whole row tiles of the plan and a ragged third."""
    if plan.kernel == TI:
        tile = plan.bm
    elif plan.kernel == NA:
        tile = 16 * (plan.wm or 4) * (plan.rb or 2)
    else:
        tile = 16 * plan.rb * max(plan.wm, 1)
    return 2 * tile + tile // 2 + 5


def boundary_ks(K):
    """k on octet, group and tail-group boundaries."""
    ks = [0, 7, 8, 127, 128, 129, 255, 256, 31, 32, 33, 64, 96, K // 2, K // 2 - 1,
          K - 129, K - 128, K - 127, K - 9, K - 8, K - 1]
    return sorted(set(k for k in ks if 0 <= k < K))


def _identity_runs(K, N, seed):
    """Lists of N column indices k, together covering every boundary k."""
    bks = boundary_ks(K)
    rng = np.random.default_rng(seed)
    runs = []
    i = 0
    while i < len(bks):
        ks = bks[i:i + N]
        i += N
        ks = ks + [int(k) for k in rng.integers(0, K, N - len(ks))]
        runs.append(ks)
    return runs


def _check_bits(C, C_ref, what):
    want = C_ref.astype(np.float16)
    bad = np.argwhere(C.view(np.uint16) != want.view(np.uint16))
    assert bad.size == 0, "%s: %d elements differ, first %s: got %r want %r" % (
        what, len(bad), tuple(bad[0]), C[tuple(bad[0])], want[tuple(bad[0])])


@pytest.mark.parametrize("name,plan,K,N,layout", CASES, ids=[c[0] for c in CASES])
def test_q_equals_z(name, plan, K, N, layout):
    plan = _resolve(plan, K, N, layout)
    M = _rows(plan)
    G = K // 128
    rng = np.random.default_rng(5)
    z = rng.integers(0, 16, (M, G), dtype=np.uint8)
    q = np.repeat(z, 128, axis=1)
    s = rng.uniform(0.002, 0.02, (M, G)).astype(np.float16)
    p = Problem(M, K, q=q, s=s, z=z)
    X = rng.standard_normal((K, N)).astype(np.float16)
    log("q==z %s M=%d K=%d N=%d plan=%s" % (name, M, K, N, plan.as_dict()))
    C = run(p, X, plan=plan, layout=layout)
    assert np.all(np.abs(C.astype(np.float64)) <= 1e-3), np.abs(C).max()


@pytest.mark.parametrize("name,plan,K,N,layout", CASES, ids=[c[0] for c in CASES])
def test_identity_columns(name, plan, K, N, layout):
    plan = _resolve(plan, K, N, layout)
    M = _rows(plan)
    Ni = N if plan.kernel == SK else min(N, 520)   # a skinny plan is built for exactly its N
    p = Problem(M, K, seed=9)
    for r, ks in enumerate(_identity_runs(K, Ni, seed=11)):
        X = np.zeros((K, Ni), dtype=np.float16)
        for n, k in enumerate(ks):
            X[k, n] = 1.0
        log("identity %s M=%d K=%d N=%d run %d plan=%s" % (name, M, K, Ni, r, plan.as_dict()))
        C = run(p, X, plan=plan, layout=layout)
        C_ref, _ = p.reference(X)
        _check_bits(C, C_ref, "identity %s k=%s" % (name, ks[:8]))


@pytest.mark.parametrize("name,plan,K,N,layout", [c for c in CASES if c[2] == 4096],
                         ids=[c[0] for c in CASES if c[2] == 4096])
def test_constant_closed_form(name, plan, K, N, layout):
    plan = _resolve(plan, K, N, layout)
    M = _rows(plan)
    G = K // 128
    q = np.full((M, K), 15, dtype=np.uint8)
    z = np.zeros((M, G), dtype=np.uint8)
    s = np.full((M, G), 0.02, dtype=np.float16)
    p = Problem(M, K, q=q, s=s, z=z)
    X = np.ones((K, N), dtype=np.float16)
    log("constant %s M=%d N=%d plan=%s" % (name, M, N, plan.as_dict()))
    C = run(p, X, plan=plan, layout=layout)
    assert np.all(C == np.float16(1229.0625)), np.unique(C)


# ---- the fused prologues (token-major): residual add + RMSNorm, and the
# gated activation.  Inputs are chosen so that the prologue's output is
# exact: h = x + r one-hot with gain 1/64 and eps 0 gives y = e_k at
# K = 4096 (mean square 2^-12, rsqrt 64); silu(16) * 0.0625 rounds to 1.0
# in fp16 and silu(16) * 0 is 0.

PROLOGUE_N = [1, 4, 8, 16, 128]


def _weights(kind, M, K, seed=9):
    G = K // 128
    rng = np.random.default_rng(seed)
    if kind == "qz":
        z = rng.integers(0, 16, (M, G), dtype=np.uint8)
        q = np.repeat(z, 128, axis=1)
        s = rng.uniform(0.002, 0.02, (M, G)).astype(np.float16)
        return Problem(M, K, q=q, s=s, z=z)
    if kind == "const":
        return Problem(M, K, q=np.full((M, K), 15, dtype=np.uint8), s=np.full((M, G), 0.02, dtype=np.float16),
                       z=np.zeros((M, G), dtype=np.uint8))
    return Problem(M, K, seed=seed)


@pytest.mark.parametrize("N", PROLOGUE_N)
def test_norm_prologue_exact(N):
    M, K = 200, 4096
    log("norm prologue gates N=%d" % N)
    rng = np.random.default_rng(N)
    # q == z: zero output whatever the activations
    p = _weights("qz", M, K)
    x = dev(rng.standard_normal((N, K)).astype(np.float16))
    r = dev(rng.standard_normal((N, K)).astype(np.float16))
    gm = dev(rng.uniform(0.1, 1.2, K).astype(np.float16))
    out, _ = B.gemm_add_rmsnorm(p.qpk, p.s_d, p.zpk, x, r, gm, 1e-6)
    torch.cuda.synchronize()
    assert np.all(np.abs(out.cpu().numpy().astype(np.float64)) <= 1e-3)
    # constant: x + r = 1, gain 1, eps 0 -> y = 1 -> 1229.0625
    p = _weights("const", M, K)
    half = dev(np.full((N, K), 0.5, dtype=np.float16))
    ones = dev(np.ones(K, dtype=np.float16))
    out, h = B.gemm_add_rmsnorm(p.qpk, p.s_d, p.zpk, half, half.clone(), ones, 0.0)
    torch.cuda.synchronize()
    assert np.all(h.cpu().numpy() == 1.0)
    assert np.all(out.cpu().numpy() == np.float16(1229.0625)), np.unique(out.cpu().numpy())
    # identity: h = e_k, gain 1/64 -> y = e_k -> fp16(Wdeq[:, k])
    p = _weights("rand", M, K)
    gm = dev(np.full(K, 1.0 / 64, dtype=np.float16))
    for ks in _identity_runs(K, N, seed=3):
        xh = np.zeros((N, K), dtype=np.float16)
        for n, k in enumerate(ks):
            xh[n, k] = 1.0
        out, _ = B.gemm_add_rmsnorm(p.qpk, p.s_d, p.zpk, dev(xh), dev(np.zeros((N, K), np.float16)), gm, 0.0)
        torch.cuda.synchronize()
        C_ref, _ = p.reference(xh.T.copy())
        _check_bits(out.cpu().numpy().T.copy(), C_ref, "norm identity N=%d k=%s" % (N, ks[:8]))


@pytest.mark.parametrize("N", PROLOGUE_N)
def test_silu_prologue_exact(N):
    M, K = 200, 4096
    log("silu prologue gates N=%d" % N)
    rng = np.random.default_rng(N)
    p = _weights("qz", M, K)
    gu = dev(rng.standard_normal((N, 2 * K)).astype(np.float16))
    out = B.gemm_silu(p.qpk, p.s_d, p.zpk, gu)
    torch.cuda.synchronize()
    assert np.all(np.abs(out.cpu().numpy().astype(np.float64)) <= 1e-3)
    # constant: gate 16, up 1/16 -> activation 1.0
    p = _weights("const", M, K)
    g = np.concatenate([np.full((N, K), 16.0), np.full((N, K), 0.0625)], axis=1).astype(np.float16)
    out = B.gemm_silu(p.qpk, p.s_d, p.zpk, dev(g))
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == np.float16(1229.0625)), np.unique(out.cpu().numpy())
    # identity: up one-hot (1/16 at k), gate 16 -> activation e_k
    p = _weights("rand", M, K)
    for ks in _identity_runs(K, N, seed=4):
        g = np.zeros((N, 2 * K), dtype=np.float16)
        g[:, :K] = 16.0
        for n, k in enumerate(ks):
            g[n, K + k] = 0.0625
        out = B.gemm_silu(p.qpk, p.s_d, p.zpk, dev(g))
        torch.cuda.synchronize()
        X = np.zeros((K, N), dtype=np.float16)
        for n, k in enumerate(ks):
            X[k, n] = 1.0
        C_ref, _ = p.reference(X)
        _check_bits(out.cpu().numpy().T.copy(), C_ref, "silu identity N=%d k=%s" % (N, ks[:8]))
