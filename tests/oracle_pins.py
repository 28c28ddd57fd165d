"""Pins of the CPU oracle against facts that do not come from the oracle.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
brute force, a closed form, an invariant or a value the PerfXLLM page states.
They are plain functions so the mutation test can run the same pins against
an oracle with a planted mistake and check that some pin fails.

``ora`` is the oracle module (``oracle.w4a16`` or a mutated copy).
"""

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# independent helpers (pure Python integers; no numpy bit tricks)

def _nibble_of_word(word, j):
    # digit j of the word written in base 16
    return (int(word) // (16 ** j)) % 16


def _brute_dequant(qpk, s, zpk, K):
    """Element-by-element Wdeq with Python ints and floats (slow)."""
    M = len(qpk)
    W = [[0.0] * K for _ in range(M)]
    for m in range(M):
        for k in range(K):
            qv = _nibble_of_word(qpk[m][k // 8], k % 8)
            g = k // 128
            zv = _nibble_of_word(zpk[m][g // 8], g % 8)
            W[m][k] = (qv - zv) * float(s[m][g])
    return W


def _brute_product(W, X):
    M, K, N = len(W), len(X), len(X[0])
    C = [[0.0] * N for _ in range(M)]
    A = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            acca = 0.0
            for k in range(K):
                p = W[m][k] * float(X[k][n])
                acc += p
                acca += abs(p)
            C[m][n] = acc
            A[m][n] = acca
    return C, A


def _words_from_codes_by_hand(codes):
    """Build uint32 words from a list of 4-bit codes by integer arithmetic."""
    words = []
    for w in range(0, len(codes), 8):
        v = 0
        for j, c in enumerate(codes[w:w + 8]):
            v += (int(c) % 16) * (16 ** j)
        words.append(v)
    return words


def _rand_case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    G = K // 128
    q = rng.integers(0, 16, (M, K), dtype=np.uint8)
    z = rng.integers(0, 16, (M, G), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, (M, G)).astype(np.float16)
    X = rng.standard_normal((K, N)).astype(np.float16)
    return q, s, z, X


# ----------------------------------------------------------------------------
# packing

def pin_pack_closed_form_words(ora):
    K = 256
    q = np.array([[k % 8 for k in range(K)]], dtype=np.uint8)
    z = np.zeros((1, 2), dtype=np.uint8)
    qpk, zpk = ora.pack(q, z)
    assert qpk.dtype == np.uint32 and qpk.shape == (1, 32)
    assert all(int(w) == 0x76543210 for w in qpk[0]), hex(int(qpk[0, 0]))
    q2 = np.zeros((1, 128), dtype=np.uint8)
    q2[0, 0] = 15
    assert int(ora.pack(q2, np.zeros((1, 1), np.uint8))[0][0, 0]) == 0x0000000F
    q3 = np.zeros((1, 128), dtype=np.uint8)
    q3[0, 7] = 15
    q3[0, 9] = 1
    w = ora.pack(q3, np.zeros((1, 1), np.uint8))[0]
    assert int(w[0, 0]) == 0xF0000000 and int(w[0, 1]) == 0x00000010
    # zeros: groups 0..7 carry codes 1..8
    zz = np.array([[1, 2, 3, 4, 5, 6, 7, 8]], dtype=np.uint8)
    qq = np.zeros((1, 8 * 128), dtype=np.uint8)
    assert int(ora.pack(qq, zz)[1][0, 0]) == 0x87654321


def pin_pack_padding_g86(ora):
    K = 11008
    G = K // 128
    assert G == 86
    rng = np.random.default_rng(5)
    z = rng.integers(0, 16, (3, G), dtype=np.uint8)
    q = rng.integers(0, 16, (3, K), dtype=np.uint8)
    qpk, zpk = ora.pack(q, z)
    assert zpk.shape == (3, 11)
    for m in range(3):
        hand = _words_from_codes_by_hand(list(z[m]))
        assert [int(v) for v in zpk[m]] == hand
        assert (int(zpk[m, 10]) >> 24) == 0          # nibbles 6, 7 are padding
        assert [int(v) for v in qpk[m]] == _words_from_codes_by_hand(list(q[m]))


def pin_pack_roundtrip(ora):
    rng = np.random.default_rng(11)
    q = rng.integers(0, 16, (7, 384), dtype=np.uint8)
    z = rng.integers(0, 16, (7, 3), dtype=np.uint8)
    qpk, zpk = ora.pack(q, z)
    q2, z2 = ora.unpack(qpk, zpk, 384)
    assert np.array_equal(q2, q) and np.array_equal(z2, z)
    words = rng.integers(0, 1 << 32, (5, 16), dtype=np.uint32)
    back = ora.pack_nibbles(ora.unpack_nibbles(words, 128))
    assert np.array_equal(back, words)
    # codes above 15 contribute their low nibble
    wide = np.array([[0x1F, 0x20, 0xFE, 3, 0, 0, 0, 0]], dtype=np.uint8)
    assert int(ora.pack_nibbles(wide)[0, 0]) == 0x00003E0F


# ----------------------------------------------------------------------------
# dequantization and product

def pin_brute_force(ora):
    for (M, K, N, seed) in [(1, 128, 1, 1), (3, 256, 2, 2), (8, 384, 3, 3),
                            (5, 128, 3, 4), (2, 384, 1, 5)]:
        q, s, z, X = _rand_case(M, K, N, seed)
        qpk, zpk = ora.pack(q, z)
        Wb = _brute_dequant(qpk.tolist(), s.astype(np.float64).tolist(),
                            zpk.tolist(), K)
        Cb, Ab = _brute_product(Wb, X.astype(np.float64).tolist())
        Wo = ora.dequant(qpk, s, zpk, K)
        assert np.array_equal(Wo, np.array(Wb)), "dequant differs from brute force"
        C, A = ora.reference(qpk, s, zpk, X)
        Cb = np.array(Cb)
        Ab = np.array(Ab)
        assert C.shape == (M, N) and A.shape == (M, N)
        assert np.all(np.abs(C - Cb) <= 1e-12 * Ab + 1e-300), "C differs"
        assert np.all(np.abs(A - Ab) <= 1e-12 * Ab + 1e-300), "A differs"


def pin_q_equals_z_gives_zero(ora):
    M, K, N = 6, 512, 3
    G = K // 128
    rng = np.random.default_rng(21)
    z = rng.integers(0, 16, (M, G), dtype=np.uint8)
    q = np.repeat(z, 128, axis=1)
    s = rng.uniform(0.002, 0.02, (M, G)).astype(np.float16)
    X = rng.standard_normal((K, N)).astype(np.float16)
    qpk, zpk = ora.pack(q, z)
    C, A = ora.reference(qpk, s, zpk, X)
    assert np.all(C == 0.0) and np.all(A == 0.0)


def pin_identity_columns(ora):
    M, K = 9, 384
    ks = [0, 7, 8, 127, 128, 255, K - 1, 200]
    q, s, z, _ = _rand_case(M, K, 1, 31)
    qpk, zpk = ora.pack(q, z)
    X = np.zeros((K, len(ks)), dtype=np.float16)
    for n, k in enumerate(ks):
        X[k, n] = 1.0
    C, A = ora.reference(qpk, s, zpk, X)
    for n, k in enumerate(ks):
        g = k // 128
        want = (q[:, k].astype(np.int64) - z[:, g].astype(np.int64)) * s[:, g].astype(np.float64)
        assert np.array_equal(C[:, n], want), "column %d (k=%d)" % (n, k)
        assert np.array_equal(A[:, n], np.abs(want))


def pin_linearity(ora):
    M, K = 4, 256
    q, s, z, _ = _rand_case(M, K, 1, 41)
    qpk, zpk = ora.pack(q, z)
    rng = np.random.default_rng(42)
    X1 = rng.standard_normal((K, 3))
    X2 = rng.standard_normal((K, 3))
    a, b = 0.75, -2.5
    C12, _ = ora.reference(qpk, s, zpk, a * X1 + b * X2)
    C1, A1 = ora.reference(qpk, s, zpk, X1)
    C2, A2 = ora.reference(qpk, s, zpk, X2)
    assert np.all(np.abs(C12 - (a * C1 + b * C2)) <= 1e-12 * (abs(a) * A1 + abs(b) * A2) + 1e-300)


def pin_constant_closed_form(ora):
    M, K = 2, 4096
    G = K // 128
    q = np.full((M, K), 15, dtype=np.uint8)
    z = np.zeros((M, G), dtype=np.uint8)
    s = np.full((M, G), 0.02, dtype=np.float16)
    assert float(s[0, 0]) == 0.0200042724609375
    X = np.ones((K, 1), dtype=np.float16)
    qpk, zpk = ora.pack(q, z)
    C, A = ora.reference(qpk, s, zpk, X)
    assert np.all(C == 1229.0625) and np.all(A == 1229.0625)


def pin_single_weight(ora):
    """One nonzero code in a non-square matrix: catches transposed operands."""
    M, K, N = 5, 384, 3
    G = K // 128
    m0, k0 = 3, 261
    q = np.zeros((M, K), dtype=np.uint8)
    q[m0, k0] = 6
    z = np.zeros((M, G), dtype=np.uint8)
    s = np.full((M, G), 0.25, dtype=np.float16)
    s[m0, k0 // 128] = 0.5
    X = np.zeros((K, N), dtype=np.float16)
    X[k0, :] = [1.0, -2.0, 0.5]
    X[k0 - 1, :] = 7.0                      # weight code 0 there: contributes 0
    qpk, zpk = ora.pack(q, z)
    C, _ = ora.reference(qpk, s, zpk, X)
    want = np.zeros((M, N))
    want[m0] = [3.0, -6.0, 1.5]
    assert np.array_equal(C, want)


def pin_group_mapping(ora):
    """Distinct power-of-two scales and known zeros per (row, group)."""
    M, K = 4, 1280
    G = K // 128
    s = np.empty((M, G), dtype=np.float16)
    z = np.empty((M, G), dtype=np.uint8)
    for m in range(M):
        for g in range(G):
            s[m, g] = 2.0 ** (-(g + m))
            z[m, g] = (3 * m + g) % 16
    q = np.full((M, K), 9, dtype=np.uint8)
    X = np.ones((K, 1), dtype=np.float16)
    qpk, zpk = ora.pack(q, z)
    C, _ = ora.reference(qpk, s, zpk, X)
    for m in range(M):
        want = 0.0
        for g in range(G):
            want += 128.0 * (9 - ((3 * m + g) % 16)) * 2.0 ** (-(g + m))
        assert C[m, 0] == want, (m, C[m, 0], want)


def pin_triangle_and_finite(ora):
    q, s, z, X = _rand_case(16, 512, 5, 51)
    qpk, zpk = ora.pack(q, z)
    C, A = ora.reference(qpk, s, zpk, X)
    assert np.all(np.isfinite(C)) and np.all(np.abs(C) <= A)


def pin_row_sampling(ora):
    q, s, z, X = _rand_case(12, 256, 2, 61)
    qpk, zpk = ora.pack(q, z)
    C, A = ora.reference(qpk, s, zpk, X)
    rows = np.array([11, 0, 5])
    Cr, Ar = ora.reference_rows(qpk, s, zpk, X, rows)
    assert np.array_equal(Cr, C[rows]) and np.array_equal(Ar, A[rows])


def pin_check_rule(ora):
    C_ref = np.array([[1.0, -2.0, 0.0]])
    A_ref = np.array([[10.0, 4.0, 0.0]])
    tol = 5e-3 * A_ref + 1e-3
    assert ora.check(C_ref + tol, C_ref, A_ref)["ok"]
    for j in range(3):                      # each element alone just outside
        over = C_ref.copy()
        over[0, j] += 1.01 * tol[0, j]
        r = ora.check(over, C_ref, A_ref)
        assert not r["ok"] and r["n_bad"] == 1, j
    bad = C_ref.copy()
    bad[0, 2] = np.nan
    r = ora.check(bad, C_ref, A_ref)
    assert not r["ok"] and r["n_nonfinite"] == 1


# ----------------------------------------------------------------------------
# format claims the page states (§3.1), stored as a cited fixture

def pin_format_claims(ora):
    with open(os.path.join(GOLDEN, "format_claims.json")) as f:
        gold = json.load(f)
    assert gold["group_size"] == ora.GROUP
    M, K = 4096, 4096
    b = ora.format_bytes(M, K)
    assert b["q"] / b["fp16"] == gold["int4_over_fp16"]
    over = (b["s"] + b["z"]) / b["fp16"]
    lo, hi = gold["scale_zero_overhead_band"]
    assert lo <= over <= hi, over
    # the whole quantized LLaMA-7B model occupies 3.7 GB; its linears alone
    # must fit inside that figure
    total = 0
    for (_, Mp, Kp) in gold["llama7b_linears_per_layer"]:
        bp = ora.format_bytes(Mp, Kp)
        total += bp["q"] + bp["s"] + bp["z"]
    total *= gold["llama7b_layers"]
    assert total < gold["model_memory_bytes"], total


# ----------------------------------------------------------------------------
# round-to-nearest quantizer (the step before the kernel)

def pin_quantizer_bounds(ora):
    rng = np.random.default_rng(71)
    W = (0.02 * rng.standard_normal((6, 512))).astype(np.float16)
    # groups of one sign, away from zero
    W[2, :128] = (0.05 + np.abs(W[2, :128].astype(np.float32))).astype(np.float16)
    W[3, 128:256] = (-0.05 - np.abs(W[3, 128:256].astype(np.float32))).astype(np.float16)
    q, s, z = ora.quantize_rtn(W)
    assert q.dtype == np.uint8 and int(q.max()) <= 15 and int(z.max()) <= 15
    qpk, zpk = ora.pack(q, z)
    Wd = ora.dequant(qpk, s, zpk, 512)
    Wf = W.astype(np.float64)
    sr = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(Wf - Wd)
    # every element within one step; unclamped codes of groups whose range
    # holds zero within half a step (plus float32 slack)
    assert np.all(err <= sr * (1 + 1e-3))
    inner = (q > 0) & (q < 15)
    assert np.all(err[inner] <= 0.5 * sr[inner] * (1 + 1e-3) + 1e-7)


def pin_quantizer_exact_grid(ora):
    """Weights already on a grid that uses codes 0 and 15 come back exactly."""
    rng = np.random.default_rng(81)
    M, K = 3, 384
    G = K // 128
    q0 = rng.integers(0, 16, (M, K), dtype=np.uint8)
    q0[:, ::128] = 0
    q0[:, 1::128] = 15
    z0 = rng.integers(0, 16, (M, G), dtype=np.uint8)
    s0 = np.array([[2.0 ** -(6 + (m + g) % 4) for g in range(G)] for m in range(M)],
                  dtype=np.float16)
    W = np.empty((M, K), dtype=np.float16)
    for m in range(M):
        for k in range(K):
            g = k // 128
            W[m, k] = (int(q0[m, k]) - int(z0[m, g])) * float(s0[m, g])
    q, s, z = ora.quantize_rtn(W)
    assert np.array_equal(s, s0) and np.array_equal(z, z0) and np.array_equal(q, q0)



# ----------------------------------------------------------------------------
# residual add + RMS normalization (§3.2 of the PerfXLLM page, first fusion)

def _norm_case(N, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((N, K)) * 2).astype(np.float16)
    r = (rng.standard_normal((N, K)) * 3).astype(np.float16)
    gamma = rng.uniform(0.5, 1.5, K).astype(np.float16)
    return x, r, gamma


def pin_norm_unit_rms(ora):
    """With unit gain and eps = 0 every output row has mean square 1 and
    keeps the signs of h."""
    x, r, _ = _norm_case(4, 384, 90)
    y, h = ora.add_rmsnorm(x, r, np.ones(384), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-12, atol=0)
    assert np.array_equal(np.sign(y), np.sign(h))


def pin_norm_one_hot(ora):
    """h = a e_j: mean square a^2 / K, so y_j = sqrt(K) sign(a) gamma_j and
    every other output is 0 (eps = 0)."""
    K = 256
    gamma = np.linspace(0.25, 2.0, K)
    for j, a in ((0, 3.0), (17, -0.5), (255, 1024.0)):
        x = np.zeros((1, K))
        x[0, j] = a
        y, _ = ora.add_rmsnorm(x, np.zeros((1, K)), gamma, 0.0)
        want = np.zeros(K)
        want[j] = np.sqrt(K) * np.sign(a) * gamma[j]
        assert np.allclose(y[0], want, rtol=1e-12, atol=1e-12)


def pin_norm_constant_row(ora):
    """h = c everywhere: y = gamma c / sqrt(c^2 + eps)."""
    K = 128
    gamma = np.arange(1, K + 1) / 64.0
    for c, eps in ((0.5, 1e-6), (-2.0, 0.25), (1e-3, 1e-6)):
        x = np.full((1, K), c / 2)
        r = np.full((1, K), c / 2)
        y, h = ora.add_rmsnorm(x, r, gamma, eps)
        assert np.allclose(h, c, rtol=0, atol=0)
        assert np.allclose(y[0], gamma * c / np.sqrt(c * c + eps), rtol=1e-12, atol=0)


def pin_norm_scale_invariance(ora):
    """eps = 0: scaling x and r by c > 0 leaves y unchanged; c < 0 flips it."""
    x, r, gamma = _norm_case(3, 256, 91)
    y, _ = ora.add_rmsnorm(x, r, gamma, 0.0)
    for c in (4.0, 1.0 / 8, -2.0):
        yc, _ = ora.add_rmsnorm(x.astype(np.float64) * c, r.astype(np.float64) * c, gamma, 0.0)
        assert np.allclose(yc, np.sign(c) * y, rtol=1e-12, atol=1e-15)


def pin_norm_zero_row(ora):
    """An all-zero stream with eps > 0 normalizes to zeros (no NaN)."""
    y, h = ora.add_rmsnorm(np.zeros((2, 128)), np.zeros((2, 128)), np.ones(128), 1e-6)
    assert np.all(y == 0) and np.all(h == 0)


def pin_norm_library(ora):
    """torch's float64 rms_norm on the summed stream (an independent
    implementation of the same definition), rows of different scales."""
    import torch
    x, r, gamma = _norm_case(5, 640, 92)
    x[3] *= np.float16(0.01)
    r[3] *= np.float16(0.01)
    h = torch.from_numpy(x).double().add(torch.from_numpy(r).double())
    for eps in (1e-6, 1e-5, 0.5):
        want = torch.nn.functional.rms_norm(h, (640,), torch.from_numpy(gamma).double(), eps).numpy()
        y, hh = ora.add_rmsnorm(x, r, gamma, eps)
        assert np.array_equal(hh, h.numpy())
        assert np.allclose(y, want, rtol=1e-12, atol=1e-14)


def pin_residual_rounding(ora):
    """fp16 rounding of the stream: ties go to the even neighbour, other
    sums to the nearest fp16 (1 + 2^-11 is half an fp16 step above 1)."""
    x = np.array([[1.0, 1.0 + 2.0 ** -10, 1.0, -3.0, 1024.0]], dtype=np.float16)
    r = np.array([[2.0 ** -11, 2.0 ** -11, 2.0 ** -11 + 2.0 ** -20, 0.5, 0.5]], dtype=np.float16)
    want = np.array([[1.0, 1.0 + 2.0 ** -9, 1.0 + 2.0 ** -10, -2.5, 1024.0]])
    got = ora.residual_fp16(x, r)
    assert got.dtype == np.float16
    assert np.array_equal(got.astype(np.float64), want)


def pin_norm_tolerance(ora):
    """The normalized-output bound admits one fp16 rounding of the exact
    value twice over and rejects a 1% error."""
    x, r, gamma = _norm_case(3, 512, 93)
    y, _ = ora.add_rmsnorm(x, r, gamma, 1e-6)
    tol = ora.norm_tolerance(y)
    assert np.all(np.abs(y.astype(np.float16).astype(np.float64) - y) <= 0.5 * tol)
    big = np.abs(y) > 0.1
    assert not np.any((np.abs(y * 1.01 - y) <= tol)[big])



# ----------------------------------------------------------------------------
# rotary encoding and decode attention (§3.2 of the PerfXLLM page, third fusion)

def pin_rope_closed_form(ora):
    """D = 2: the pair turns by pos radians; D = 4 with base 16: the second
    pair turns by pos / 4; position 0 is the identity."""
    for p in (0, 1, 3, 100):
        assert np.allclose(ora.rope([1.0, 0.0], p), [np.cos(p), np.sin(p)], rtol=0, atol=1e-15)
        assert np.allclose(ora.rope([0.0, 1.0], p), [-np.sin(p), np.cos(p)], rtol=0, atol=1e-15)
        assert np.allclose(ora.rope([0.0, 0.0, 1.0, 0.0], p, base=16.0),
                           [0.0, 0.0, np.cos(p / 4), np.sin(p / 4)], rtol=0, atol=1e-15)
        assert np.allclose(ora.rope([0.0, 1.0, 0.0, 0.0], p, base=16.0),
                           [-np.sin(p), np.cos(p), 0.0, 0.0], rtol=0, atol=1e-15)
    x = np.random.default_rng(94).standard_normal((3, 128))
    assert np.array_equal(ora.rope(x, 0), x)


def pin_rope_complex(ora):
    """The pairs as complex numbers x[2i] + i x[2i+1], multiplied by
    exp(i pos base^(-2i/D)); pair norms are kept."""
    rng = np.random.default_rng(95)
    D = 128
    x = rng.standard_normal((4, D))
    pos = np.array([0, 1, 17, 2047])
    z = x[:, 0::2] + 1j * x[:, 1::2]
    ang = pos[:, None] * np.power(10000.0, -np.arange(0, D, 2) / D)[None, :]
    w = z * np.exp(1j * ang)
    got = ora.rope(x, pos)
    assert np.allclose(got[:, 0::2], w.real, rtol=0, atol=1e-12)
    assert np.allclose(got[:, 1::2], w.imag, rtol=0, atol=1e-12)
    assert np.allclose(np.hypot(got[:, 0::2], got[:, 1::2]), np.abs(z), rtol=1e-13)


def pin_rope_relative_position(ora):
    """q . k after encoding depends on the positions only through their
    difference."""
    rng = np.random.default_rng(96)
    q, k = rng.standard_normal((2, 128))
    for m, n, t in ((5, 2, 100), (0, 9, 33), (700, 700, 1)):
        a = ora.rope(q, m) @ ora.rope(k, n)
        b = ora.rope(q, m + t) @ ora.rope(k, n + t)
        assert abs(a - b) <= 1e-10 * (1 + abs(a))


def _attn_case(B, H, D, S, seed):
    rng = np.random.default_rng(seed)
    qkv = rng.standard_normal((B, 3 * H * D)).astype(np.float16)
    kc = rng.standard_normal((B, H, S, D)).astype(np.float16)
    vc = rng.standard_normal((B, H, S, D)).astype(np.float16)
    return qkv, kc, vc


def pin_attention_first_token(ora):
    """At position 0 the only key is the new one: out = fp16(v), whatever q
    and k are; the stored key is rope(k, 0) = k."""
    qkv, kc, vc = _attn_case(2, 3, 16, 4, 97)
    out, A, kn, vn = ora.decode_attention(qkv, kc, vc, [0, 0], 3, 16)
    v = qkv[:, 2 * 48:].astype(np.float64)
    assert np.array_equal(out, v) and np.array_equal(A, np.abs(v))
    assert np.array_equal(kn.reshape(2, 48), qkv[:, 48:96].astype(np.float64))


def pin_attention_uniform(ora):
    """q = 0: every score is 0, so out is the mean of the p + 1 values and A
    the mean of their magnitudes."""
    H, D, S = 2, 8, 12
    qkv, kc, vc = _attn_case(3, H, D, S, 98)
    qkv[:, :H * D] = 0
    pos = [1, 7, 11]
    out, A, _, _ = ora.decode_attention(qkv, kc, vc, pos, H, D)
    for b, p in enumerate(pos):
        V = np.concatenate([vc[b, :, :p].astype(np.float64),
                            qkv[b, 2 * H * D:].astype(np.float64).reshape(H, 1, D)], axis=1)
        assert np.allclose(out[b], V.mean(axis=1).reshape(-1), rtol=1e-13, atol=1e-15)
        assert np.allclose(A[b], np.abs(V).mean(axis=1).reshape(-1), rtol=1e-13, atol=1e-15)


def pin_attention_two_keys_closed_form(ora):
    """D = 2, position 1: q = k = (1, 0) both turn by 1 radian, and the cached
    key (cos 1, sin 1) equals the new one up to its fp16 rounding, so the two
    scores match and out is the mean of the two values."""
    c1 = np.float16(np.cos(1.0))
    s1 = np.float16(np.sin(1.0))
    qkv = np.array([[1.0, 0.0, 1.0, 0.0, 3.0, -1.0]], dtype=np.float16)
    kc = np.array([[[[c1, s1], [0, 0]]]], dtype=np.float16)
    vc = np.array([[[[1.0, 5.0], [0, 0]]]], dtype=np.float16)
    out, _, kn, _ = ora.decode_attention(qkv, kc, vc, [1], 1, 2)
    assert np.allclose(kn[0, 0], [np.cos(1.0), np.sin(1.0)], rtol=0, atol=1e-15)
    assert np.allclose(out[0], [2.0, 2.0], rtol=0, atol=1e-12)


def pin_attention_dominant_key(ora):
    """A cached key along q, 40x longer than the others: its value wins."""
    H, D, S = 1, 16, 9
    qkv, kc, vc = _attn_case(1, H, D, S, 99)
    p = 6
    qr = ora.rope(qkv[0, :D].astype(np.float64), p)
    kc[0, 0, 3] = (qr / np.linalg.norm(qr) * 40).astype(np.float16)
    out, _, _, _ = ora.decode_attention(qkv, kc, vc, [p], H, D)
    assert np.allclose(out[0], vc[0, 0, 3].astype(np.float64), rtol=0, atol=1e-6)


def pin_attention_library(ora):
    """torch's float64 scaled_dot_product_attention over the rotated query and
    the keys and values the step attends to (default scale 1/sqrt(D))."""
    import torch
    H, D, S = 4, 32, 20
    qkv, kc, vc = _attn_case(3, H, D, S, 100)
    pos = [0, 9, 19]
    out, _, kn, vn = ora.decode_attention(qkv, kc, vc, pos, H, D)
    for b, p in enumerate(pos):
        q = torch.from_numpy(ora.rope(qkv[b, :H * D].astype(np.float64).reshape(H, D), p))
        K = torch.cat([torch.from_numpy(kc[b, :, :p].astype(np.float64)),
                       torch.from_numpy(kn[b].astype(np.float16).astype(np.float64))[:, None, :]], dim=1)
        V = torch.cat([torch.from_numpy(vc[b, :, :p].astype(np.float64)),
                       torch.from_numpy(vn[b].astype(np.float16).astype(np.float64))[:, None, :]], dim=1)
        want = torch.nn.functional.scaled_dot_product_attention(q[:, None, :], K, V)[:, 0, :].reshape(-1)
        assert np.allclose(out[b], want.numpy(), rtol=1e-12, atol=1e-13)


def pin_rope_tolerance(ora):
    """The stored-key bound admits one fp16 rounding and rejects 1%."""
    rng = np.random.default_rng(101)
    x = rng.standard_normal((64, 128))
    y = ora.rope(x, 1234)
    pn = np.repeat(np.hypot(y[:, 0::2], y[:, 1::2]), 2, axis=1)
    tol = ora.rope_tolerance(y, pn)
    assert np.all(np.abs(y.astype(np.float16).astype(np.float64) - y) <= tol)
    big = np.abs(y) > 0.1
    assert not np.any((np.abs(0.01 * y) <= tol)[big])



# ----------------------------------------------------------------------------
# gated MLP activation (the decoder layer's silu(gate) * up)

def pin_silu_mul_closed_forms(ora):
    """silu(0) = 0, silu(g) - silu(-g) = g (the logistic function's symmetry),
    silu(g) -> g for large g and -> 0 for very negative g; gate and up are the
    first and second halves of a row."""
    g = np.array([0.0, 1.0, -1.0, 2.5, 40.0, -40.0])
    one = np.ones_like(g)
    gu = np.stack([np.concatenate([g, one]), np.concatenate([-g, one])])
    a = ora.silu_mul(gu)
    assert a[0, 0] == 0.0
    assert np.allclose(a[0] - a[1], g, rtol=0, atol=1e-12)
    assert abs(a[0, 4] - 40.0) < 1e-12 and abs(a[0, 5]) < 1e-15
    assert abs(a[0, 1] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
    up = np.arange(1.0, 7.0)
    a2 = ora.silu_mul(np.concatenate([np.full(6, 1.0), up])[None, :])
    assert np.allclose(a2[0], up / (1.0 + np.exp(-1.0)), rtol=1e-15)


def pin_silu_mul_library(ora):
    """torch's float64 silu times the up half."""
    import torch
    rng = np.random.default_rng(102)
    gu = (rng.standard_normal((3, 512)) * 4).astype(np.float16)
    t = torch.from_numpy(gu.astype(np.float64))
    want = (torch.nn.functional.silu(t[:, :256]) * t[:, 256:]).numpy()
    assert np.allclose(ora.silu_mul(gu), want, rtol=1e-14, atol=1e-300)


def pin_silu_mul_tolerance(ora):
    rng = np.random.default_rng(103)
    ref = ora.silu_mul(rng.standard_normal((4, 256)) * 3)
    tol = ora.silu_mul_tolerance(ref)
    assert np.all(np.abs(ref.astype(np.float16).astype(np.float64) - ref) <= tol)
    big = np.abs(ref) > 0.1
    assert not np.any((np.abs(0.01 * ref) <= tol)[big])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
