"""Fused decode attention against the oracle: the output element by element
(|out - ref| <= 5e-3 * sum_j p_j |V_j| + 1e-3), the stored key within the
rotary tolerance, the stored value bit for bit, every other cache entry
untouched; single and split workgroup spans, ragged positions, the first
position, positions out of range, two steps in a row."""

import numpy as np
import pytest
import torch

import oracle.w4a16 as ora
from gemm_w4a16_group_amd import binding as B
from gemm_w4a16_group_amd import inputs
from gpu_util import dev, log

pytestmark = pytest.mark.gpu

D = 128


def check_step(qkv, kc, vc, pos, kc_gpu, vc_gpu, out_gpu, H, what):
    """kc, vc: the caches before the step (host); *_gpu: after it."""
    Bn = qkv.shape[0]
    ref, A, k_new, v_new = ora.decode_attention(qkv, kc, vc, pos, H, D)
    err = np.abs(out_gpu.astype(np.float64) - ref)
    tol = ora.tolerance(A)
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d bad outputs, max err/tol %.3g" % (what, int(bad.sum()), float(np.max(err / tol)))
    kc_exp, vc_exp = kc.copy(), vc.copy()
    for b in range(Bn):
        p = int(pos[b])
        pn = np.repeat(np.hypot(k_new[b][:, 0::2], k_new[b][:, 1::2]), 2, axis=1)
        kerr = np.abs(kc_gpu[b, :, p].astype(np.float64) - k_new[b])
        assert np.all(kerr <= ora.rope_tolerance(k_new[b], pn)), "%s: stored key of sequence %d" % (what, b)
        assert np.array_equal(vc_gpu[b, :, p], v_new[b].astype(np.float16)), "%s: stored value %d" % (what, b)
        kc_exp[b, :, p] = kc_gpu[b, :, p]
        vc_exp[b, :, p] = vc_gpu[b, :, p]
    assert np.array_equal(kc_gpu.view(np.uint16), kc_exp.view(np.uint16)), what + ": other keys changed"
    assert np.array_equal(vc_gpu.view(np.uint16), vc_exp.view(np.uint16)), what + ": other values changed"
    return k_new, v_new


def run_step(qkv, kc, vc, pos, max_len=None):
    kd, vd = dev(kc), dev(vc)
    out = B.decode_attention(dev(qkv), kd, vd, dev(np.asarray(pos, dtype=np.int32)), max_len=max_len)
    torch.cuda.synchronize()
    return out.cpu().numpy(), kd.cpu().numpy(), vd.cpu().numpy()


CASES = [
    # (B, H, S, max_len or None, positions)
    (1, 1, 16, None, [15]),
    (1, 4, 64, None, [0]),
    (3, 8, 300, None, [0, 150, 299]),
    (5, 2, 1000, 600, [599, 1, 17, 0, 300]),
    (1, 32, 2048, None, [2047]),
    (2, 32, 4096, None, [4095, 1000]),
    (16, 32, 512, None, list(range(7, 512, 32))),
    (4, 32, 2048, 1500, [1499, 64, 777, 1024]),
    (2, 3, 130, None, [128, 129]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_H%d_S%d_L%s" % (c[0], c[1], c[2], c[3]))
def test_decode_attention(case):
    Bn, H, S, max_len, pos = case
    log("decode_attention %s" % (case[:4],))
    qkv, kc, vc = inputs.attention_inputs(Bn, H, D, S, wid=600 + S + Bn)
    out, kg, vg = run_step(qkv, kc, vc, pos, max_len)
    check_step(qkv, kc, vc, pos, kg, vg, out, H, str(case[:4]))


def test_decode_attention_positions_out_of_range():
    """A position outside [0, max_len) gives NaN outputs for its sequence and
    leaves its cache alone; the other sequences are unaffected."""
    Bn, H, S = 4, 4, 256
    qkv, kc, vc = inputs.attention_inputs(Bn, H, D, S, wid=640)
    pos = [10, -1, 200, 100]
    out, kg, vg = run_step(qkv, kc, vc, pos, max_len=200)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
    for b in (1, 2):
        assert np.array_equal(kg[b], kc[b]) and np.array_equal(vg[b], vc[b])
    keep = [0, 3]
    check_step(qkv[keep], kc[keep], vc[keep], [pos[b] for b in keep], kg[keep], vg[keep], out[keep], H,
               "in-range sequences")


def test_decode_attention_two_steps():
    """Step p then p + 1 on the same device caches; the oracle replays both
    steps on its own caches (fp16 roundings of its own stored entries)."""
    Bn, H, S = 2, 8, 1024
    qkv1, kc, vc = inputs.attention_inputs(Bn, H, D, S, wid=650)
    qkv2, _, _ = inputs.attention_inputs(Bn, H, D, 1, wid=651)
    pos1 = np.array([500, 1000], dtype=np.int32)
    kd, vd = dev(kc), dev(vc)
    o1 = B.decode_attention(dev(qkv1), kd, vd, dev(pos1)).cpu().numpy()
    o2 = B.decode_attention(dev(qkv2), kd, vd, dev(pos1 + 1)).cpu().numpy()
    torch.cuda.synchronize()
    ref1, A1, kn1, vn1 = ora.decode_attention(qkv1, kc, vc, pos1, H, D)
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(Bn):
        kc2[b, :, pos1[b]] = kn1[b].astype(np.float16)
        vc2[b, :, pos1[b]] = vn1[b].astype(np.float16)
    ref2, A2, _, _ = ora.decode_attention(qkv2, kc2, vc2, pos1 + 1, H, D)
    for o, r, a, name in ((o1, ref1, A1, "step 1"), (o2, ref2, A2, "step 2")):
        err = np.abs(o.astype(np.float64) - r)
        assert np.all(err <= ora.tolerance(a)), name


SHAPES = [(16, 4), (32, 4), (64, 4), (16, 8), (32, 8), (64, 8), (16, 16)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "kpw%d_w%d" % s)
def test_decode_attention_shapes(shape):
    """Every workgroup shape on a split case and a single-workgroup case."""
    for Bn, H, S, pos in ((2, 8, 1500, [1499, 700]), (1, 4, 40, [39]), (3, 2, 3000, [2999, 0, 1024])):
        log("decode_attention shape %s B=%d S=%d" % (shape, Bn, S))
        qkv, kc, vc = inputs.attention_inputs(Bn, H, D, S, wid=660 + S)
        kd, vd = dev(kc), dev(vc)
        out = B.decode_attention(dev(qkv), kd, vd, dev(np.asarray(pos, dtype=np.int32)), shape=shape)
        torch.cuda.synchronize()
        check_step(qkv, kc, vc, pos, kd.cpu().numpy(), vd.cpu().numpy(), out.cpu().numpy(), H,
                   "shape %s B=%d" % (shape, Bn))
