"""Plain float64 oracle for the W4A16 group-quantized linear layer.

TEST INFRASTRUCTURE: only tests, the smoke check and the bench's CPU-baseline
leg use this module.  It imports numpy and nothing else.

Notation follows the PerfXLLM page (3532n.com/d/2322131), §3.3 item 1: the
product is C[m, n] = A[m, k] . B[k, n], where A is the dequantized weight
matrix (called W or Wdeq below) and B the fp16 activations (called X).
The residual add + RMS normalization that feeds the projections (§3.2, first
fusion) is at the end of the module, with its tolerance.
"""

import numpy as np

# §3.1 of the PerfXLLM page: one scale and one zero per 128 weights.
GROUP = 128


def _groups(K):
    if K % GROUP:
        raise ValueError("K must be a multiple of %d, got %d" % (GROUP, K))
    return K // GROUP


def pack_nibbles(v):
    """Pack 4-bit codes along the last axis, eight per uint32, low nibble first.

    ``v`` is an integer array [R, L]; only the low four bits of each entry are
    kept.  The result is uint32 [R, ceil(L / 8)]; nibble j of word w holds
    v[:, 8 * w + j] in bits 4j .. 4j + 3.  Nibbles past L are zero.
    """
    v = np.asarray(v)
    if v.ndim != 2:
        raise ValueError("pack_nibbles wants a 2-D array")
    R, L = v.shape
    W = (L + 7) // 8
    padded = np.zeros((R, W * 8), dtype=np.uint32)
    padded[:, :L] = v.astype(np.uint32) & np.uint32(0xF)
    words = np.zeros((R, W), dtype=np.uint32)
    for j in range(8):
        words |= padded[:, j::8] << np.uint32(4 * j)
    return words


def unpack_nibbles(words, L):
    """Inverse of ``pack_nibbles``: uint32 [R, W] -> uint8 [R, L]."""
    words = np.asarray(words, dtype=np.uint32)
    if words.ndim != 2:
        raise ValueError("unpack_nibbles wants a 2-D array")
    R, W = words.shape
    if W * 8 < L:
        raise ValueError("%d words cannot hold %d nibbles" % (W, L))
    out = np.empty((R, W * 8), dtype=np.uint8)
    for j in range(8):
        out[:, j::8] = (words >> np.uint32(4 * j)) & np.uint32(0xF)
    return out[:, :L]


def pack(q, z):
    """Pack weight codes q [M, K] and zero codes z [M, K/128].

    Returns (qpk uint32 [M, K/8], zpk uint32 [M, ceil(G/8)]).  The zero is read
    as a 4-bit code packed like the weights, along the group axis.
    """
    q = np.asarray(q)
    z = np.asarray(z)
    M, K = q.shape
    G = _groups(K)
    if z.shape != (M, G):
        raise ValueError("z must be [M, K/128] = %r, got %r" % ((M, G), z.shape))
    return pack_nibbles(q), pack_nibbles(z)


def unpack(qpk, zpk, K):
    """Return (q uint8 [M, K], z uint8 [M, K/128]) from the packed arrays."""
    G = _groups(K)
    return unpack_nibbles(qpk, K), unpack_nibbles(zpk, G)


def dequant(qpk, s, zpk, K, rows=None):
    """Wdeq[m, k] = (q[m, k] - z[m, k // 128]) * s[m, k // 128] in float64.

    §3.1 of the PerfXLLM page gives int4 weights with a scale and a zero per
    group of 128; the zero is taken as an integer code subtracted before the
    scale is applied.  ``rows`` optionally selects a subset of rows.
    """
    qpk = np.asarray(qpk, dtype=np.uint32)
    zpk = np.asarray(zpk, dtype=np.uint32)
    s = np.asarray(s)
    if rows is not None:
        qpk, zpk, s = qpk[rows], zpk[rows], s[rows]
    q, z = unpack(qpk, zpk, K)
    G = K // GROUP
    if s.shape != (q.shape[0], G):
        raise ValueError("s must be [M, K/128], got %r" % (s.shape,))
    qf = q.astype(np.float64).reshape(q.shape[0], G, GROUP)
    zf = z.astype(np.float64)[:, :, None]
    sf = s.astype(np.float64)[:, :, None]
    return ((qf - zf) * sf).reshape(q.shape[0], K)


def _block_rows(K, N):
    # keep one dequantized block (plus its |.|) near 256 MB of float64
    return max(1, (1 << 25) // max(K, 1))


def reference(qpk, s, zpk, X):
    """C = Wdeq @ X and A = |Wdeq| @ |X| in float64 (§3.3 items 1 and 2).

    X is [K, N] (any float dtype; N = 1 is the GEMV of item 2).  The work is
    done in row blocks so large matrices fit in host memory; the blocking
    changes nothing but which rows are in flight.
    """
    X = np.asarray(X)
    if X.ndim != 2:
        raise ValueError("X must be [K, N]")
    K, N = X.shape
    M = np.asarray(qpk).shape[0]
    Xf = X.astype(np.float64)
    Xa = np.abs(Xf)
    C = np.empty((M, N), dtype=np.float64)
    A = np.empty((M, N), dtype=np.float64)
    step = _block_rows(K, N)
    for r0 in range(0, M, step):
        rows = slice(r0, min(M, r0 + step))
        W = dequant(qpk, s, zpk, K, rows=rows)
        C[rows] = W @ Xf
        A[rows] = np.abs(W) @ Xa
    return C, A


def reference_rows(qpk, s, zpk, X, rows):
    """``reference`` restricted to the given row indices (for sampled checks)."""
    rows = np.asarray(rows)
    X = np.asarray(X)
    K = X.shape[0]
    W = dequant(qpk, s, zpk, K, rows=rows)
    Xf = X.astype(np.float64)
    return W @ Xf, np.abs(W) @ np.abs(Xf)


def tolerance(A):
    """Per-element bound 5e-3 * sum_k |Wdeq[m,k] X[k,n]| + 1e-3."""
    return 5e-3 * np.asarray(A, dtype=np.float64) + 1e-3


def check(C_test, C_ref, A_ref):
    """Compare a result with the oracle element by element.

    Returns a dict with ``ok`` (every element within ``tolerance``),
    ``max_err_over_tol``, ``max_abs_err``, ``max_rel_to_A`` (over elements
    with A > 0), ``n_bad`` and ``n_nonfinite``.
    """
    Ct = np.asarray(C_test, dtype=np.float64)
    err = np.abs(Ct - C_ref)
    tol = tolerance(A_ref)
    finite = np.isfinite(Ct)
    ratio = np.where(finite, err / tol, np.inf)
    nz = A_ref > 0
    rel = float(np.max(err[nz] / A_ref[nz])) if np.any(nz & finite) else 0.0
    n_bad = int(np.count_nonzero(~(ratio <= 1.0)))
    return {
        "ok": n_bad == 0,
        "max_err_over_tol": float(np.max(ratio)) if ratio.size else 0.0,
        "max_abs_err": float(np.max(np.where(finite, err, np.inf))) if err.size else 0.0,
        "max_rel_to_A": rel,
        "n_bad": n_bad,
        "n_nonfinite": int(np.count_nonzero(~finite)),
    }


def quantize_rtn(W):
    """Round-to-nearest asymmetric group quantizer, W [M, K] -> (q, s, z).

    The step that produces the kernel's inputs from fp16 weights (§3.1 of
    the PerfXLLM page quantizes weights only, to int4, g = 128).  AWQ's
    activation-aware scale search needs calibration data and is not modelled;
    this is the plain min/max form:

      lo, hi = min(group min, 0) and max(group max, 0)  (float32)
      s      = fp16( max(hi - lo, 1e-5) / 15 )          (float32 divide)
      z      = clamp(rint(-lo / s), 0, 15)              (float32 divide)
      q      = clamp(rint(w / s) + z, 0, 15)            (float32 divide)

    The range is widened to hold 0, so that the zero code stays in [0, 15]
    for groups of one sign.  rint rounds half to even.  The codes are
    integer decisions taken in
    float32 from the stored fp16 scale, the precision the device kernel
    uses, so both sides decide alike.
    """
    W = np.asarray(W)
    M, K = W.shape
    G = _groups(K)
    w = W.astype(np.float32).reshape(M, G, GROUP)
    lo = np.minimum(w.min(axis=2), np.float32(0.0))
    hi = np.maximum(w.max(axis=2), np.float32(0.0))
    rng = np.maximum(hi - lo, np.float32(1e-5))
    s16 = (rng / np.float32(15.0)).astype(np.float32).astype(np.float16)
    s32 = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / s32), 0, 15).astype(np.float32)
    q = np.clip(np.rint(w / s32[:, :, None]) + z[:, :, None], 0, 15)
    return q.reshape(M, K).astype(np.uint8), s16, z.astype(np.uint8)


def format_bytes(M, K):
    """Storage of the packed format: dict of byte counts for one M x K matrix.

    ``q`` = M*K/2 (int4), ``s`` = 2*M*G (fp16), ``z`` = M*G/2 (4-bit codes,
    counted without word padding), ``fp16`` = 2*M*K for the unquantized matrix.
    """
    G = _groups(K)
    return {"q": M * K // 2, "s": 2 * M * G, "z": M * G // 2, "fp16": 2 * M * K}


def add_rmsnorm(x, r, gamma, eps):
    """Residual add followed by RMS normalization, token-major, in float64.

    §3.2 of the PerfXLLM page (operator fusion, first part) runs the residual
    network's addition and the normalization that follows it as one
    operator.  The page does not name the normalization; LLaMA's is RMSNorm,
    the reading taken here: per token, no mean subtraction, no bias, a
    learned gain per hidden channel.

      h[n, k] = x[n, k] + r[n, k]
      y[n, k] = h[n, k] / sqrt(mean_k h[n, k]^2 + eps) * gamma[k]

    x, r: [N, K] (fp16 or float), gamma: [K], eps >= 0.  Returns (y, h) in
    float64.  The residual stream is stored in fp16: ``residual_fp16`` gives
    the stored h, and the normalization of the stored stream is
    ``add_rmsnorm(h16, 0, gamma, eps)``.
    """
    h = np.asarray(x, dtype=np.float64) + np.asarray(r, dtype=np.float64)
    if h.ndim != 2:
        raise ValueError("x and r must be [N, K]")
    ms = np.mean(h * h, axis=1)
    y = h / np.sqrt(ms + float(eps))[:, None] * np.asarray(gamma, dtype=np.float64)[None, :]
    return y, h


def residual_fp16(x, r):
    """The stored residual stream fp16(x + r): the exact sum (float64 holds
    the sum of two fp16 values exactly) rounded to nearest, ties to even."""
    return (np.asarray(x, dtype=np.float64) + np.asarray(r, dtype=np.float64)).astype(np.float16)


def norm_tolerance(y_ref):
    """Per-element bound on a normalized fp16 output: 2e-3 * |y| + 1e-6.

    Budget (relative): fp16 rounding of the stored stream h (2^-11), of the
    output (2^-11), a float32 mean of squares and reciprocal square root
    (below 2e-5 at K <= 2^16): about 1.0e-3, doubled; the absolute floor
    covers outputs in the fp16 subnormal range (spacing 6e-8)."""
    return 2e-3 * np.abs(np.asarray(y_ref, dtype=np.float64)) + 1e-6


def rope(x, pos, base=10000.0):
    """Rotary position encoding of the last axis of x (length D, even).

    §3.2 of the PerfXLLM page fuses the rotary encoding of Q and K into the
    attention operator without defining it; read here as LLaMA's: the
    channel pairs (2i, 2i + 1) of a head are rotated by the angle
    pos * base^(-2i / D):

      out[2i]     = x[2i] cos(a_i) - x[2i + 1] sin(a_i)
      out[2i + 1] = x[2i] sin(a_i) + x[2i + 1] cos(a_i)

    pos broadcasts against x[..., 0].  float64 throughout.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % 2:
        raise ValueError("the head dimension must be even")
    i = np.arange(D // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / D)
    a = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(a), np.sin(a)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def decode_attention(qkv, k_cache, v_cache, pos, H, D, base=10000.0, scale=None):
    """One decode step of multi-head attention per sequence, in float64.

    §3.2 of the PerfXLLM page, third fusion: the rotary encoding of Q and K,
    the two products QK^T and PV, and the softmax between them.  For each
    sequence b with its new token at position p = pos[b] (0-based):

      q, k, v = the head slices of qkv[b] = [q | k | v], each [H, D]
      q' = rope(q, p);  k' = fp16(rope(k, p))    (k' is stored in the cache)
      keys j = 0 .. p: K_j = k_cache[b, :, j] for j < p, K_p = k'
                       V_j = v_cache[b, :, j] for j < p, V_p = fp16(v)
      s_j = scale * q' . K_j  (scale = 1 / sqrt(D) by default)
      out[b, h] = sum_j softmax(s)_j V_j

    qkv: [B, 3 H D]; k_cache, v_cache: [B, H, S, D]; pos: [B] ints with
    0 <= p < S.  Returns (out [B, H D], A [B, H D], k_new [B, H, D],
    v_new [B, H, D]), where A = sum_j softmax(s)_j |V_j| bounds the error
    of out, and k_new / v_new are the float64 entries the step stores at
    position p (the stored values are their fp16 roundings).
    """
    qkv = np.asarray(qkv, dtype=np.float64)
    B = qkv.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, H * D))
    A = np.zeros((B, H * D))
    k_new = np.zeros((B, H, D))
    v_new = np.zeros((B, H, D))
    for b in range(B):
        p = int(pos[b])
        q = qkv[b, 0:H * D].reshape(H, D)
        k = qkv[b, H * D:2 * H * D].reshape(H, D)
        v = qkv[b, 2 * H * D:3 * H * D].reshape(H, D)
        qr = rope(q, p, base)
        kr = rope(k, p, base)
        k_new[b], v_new[b] = kr, v
        Kc = np.asarray(k_cache[b, :, :p], dtype=np.float64)
        Vc = np.asarray(v_cache[b, :, :p], dtype=np.float64)
        Kall = np.concatenate([Kc, kr.astype(np.float16).astype(np.float64)[:, None, :]], axis=1)
        Vall = np.concatenate([Vc, v.astype(np.float16).astype(np.float64)[:, None, :]], axis=1)
        for h in range(H):
            s = scale * (Kall[h] @ qr[h])
            w = np.exp(s - s.max())
            w /= w.sum()
            out[b, h * D:(h + 1) * D] = w @ Vall[h]
            A[b, h * D:(h + 1) * D] = w @ np.abs(Vall[h])
    return out, A, k_new, v_new


def rope_tolerance(ref, pair_norm):
    """Bound on a stored fp16 rotated key: half an fp16 step (2^-11 |ref|),
    float32 rotation of the pair (1e-6 of its norm) and the fp16 subnormal
    half-spacing (6e-8)."""
    return 2.0 ** -11 * np.abs(ref) + 1e-6 * pair_norm + 6e-8


def silu_mul(gu):
    """The gated activation of LLaMA's MLP on the fused gate/up projection's
    output, in float64: gu is [N, 2 I] with the gate in columns 0 .. I - 1
    and the up projection in I .. 2 I - 1 (the fused 22016 = 2 x 11008 rows
    of the gate/up weight, gate rows first);

      act[n, i] = silu(g) * u,  silu(g) = g / (1 + exp(-g)).

    The pages do not describe the MLP; this is the LLaMA-7B reading.
    """
    gu = np.asarray(gu, dtype=np.float64)
    I = gu.shape[1] // 2
    if gu.shape[1] != 2 * I:
        raise ValueError("gu must have an even number of columns")
    g, u = gu[:, :I], gu[:, I:]
    return g / (1.0 + np.exp(-g)) * u


def silu_mul_tolerance(ref):
    """Bound on an fp16 activation: one fp16 rounding (2^-11 |ref|), float32
    exp and divide (below 1e-6 relative), doubled; absolute floor 1e-6."""
    return 1e-3 * np.abs(np.asarray(ref, dtype=np.float64)) + 1e-6
