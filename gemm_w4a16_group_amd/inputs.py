"""Seeded synthetic inputs for the W4A16 linear layer.

This module only draws random numbers.  It holds none of the layer's
arithmetic (no packing, no dequantization, no products), so the HIP path and
the CPU oracle can both be fed from it without sharing any of the method.

Distributions (the quantized LLaMA-7B linears of the PerfXLLM page, §2 and
§3.1: int4 codes, one scale and one zero per 128 weights):

* q: uniform integer codes in [0, 15], shape [M, K];
* z: uniform integer codes in [0, 15], shape [M, K / 128];
* s: uniform in [0.002, 0.02], drawn in float64 and rounded to fp16;
* X: standard normal, drawn in float32 and rounded to fp16, shape [K, N].

Seeds are numpy PCG64 streams keyed by (workload id, layer, projection,
stream); weights use stream 0 and activations stream 1 + N, so one weight
matrix serves a whole sweep over N with fresh activations per N.
"""

import numpy as np

GROUP = 128

# LLaMA-7B linear shapes (M = output rows, K = reduction length).  The page
# fuses the three QKV products into one (§3.2), giving M = 3 * 4096.
LLAMA7B_PROJ = (
    ("qkv", 12288, 4096),
    ("o_proj", 4096, 4096),
    ("gate_up", 22016, 4096),
    ("down", 4096, 11008),
)

# Named workloads.  ``wid`` is the seed key of each workload.
WORKLOADS = {
    "gemv_4096x4096": {"wid": 1, "shapes": [("w", 4096, 4096)], "N": [1]},
    "llama7b_decode_linears": {"wid": 2, "shapes": list(LLAMA7B_PROJ), "N": [1]},
    "small_n_12288x4096": {"wid": 3, "shapes": [("w", 12288, 4096)],
                           "N": [1, 2, 4, 8, 16, 32]},
    "large_n_12288x4096": {"wid": 4, "shapes": [("w", 12288, 4096)],
                           "N": [64, 128, 256, 512, 1024, 2048, 4096]},
    "llama7b_stack_32x4": {"wid": 5, "shapes": list(LLAMA7B_PROJ), "N": [1, 16],
                           "layers": 32},
}


def weight_rng(wid, layer, proj):
    return np.random.default_rng([wid, layer, proj, 0])


def act_rng(wid, layer, proj, N):
    return np.random.default_rng([wid, layer, proj, 1 + N])


def weights(M, K, wid=0, layer=0, proj=0):
    """(q uint8 [M, K], s float16 [M, K/128], z uint8 [M, K/128])."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    rng = weight_rng(wid, layer, proj)
    G = K // GROUP
    q = rng.integers(0, 16, (M, K), dtype=np.uint8)
    z = rng.integers(0, 16, (M, G), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, (M, G)).astype(np.float16)
    return q, s, z


def raw_q_words(M, K, wid=0, layer=0, proj=0):
    """Uniform random uint32 words [M, K/8] for the weight codes.

    Eight independent uniform 4-bit codes per word have the same law as a
    uniform 32-bit word, so large stacks draw the packed words directly
    instead of 8x as many bytes of codes.  Scales and zeros come from
    ``scales_zeros`` with the same seed key.
    """
    rng = weight_rng(wid, layer, proj)
    return rng.integers(0, 1 << 32, (M, K // 8), dtype=np.uint32)


def scales_zeros(M, K, wid=0, layer=0, proj=0):
    """(s float16 [M, K/128], z uint8 [M, K/128]) on their own stream."""
    rng = np.random.default_rng([wid, layer, proj, 2])
    G = K // GROUP
    z = rng.integers(0, 16, (M, G), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, (M, G)).astype(np.float16)
    return s, z


def activations(K, N, wid=0, layer=0, proj=0):
    """X float16 [K, N], standard normal rounded to fp16."""
    rng = act_rng(wid, layer, proj, N)
    return rng.standard_normal((K, N), dtype=np.float32).astype(np.float16)


def uniform_codes(shape, seed):
    """Uniform integer codes in [0, 15] (generic helper for tests)."""
    return np.random.default_rng(seed).integers(0, 16, shape, dtype=np.uint8)


def fp16_weights(M, K, wid=0, layer=0, proj=0, sigma=0.02, outliers=1e-3):
    """Unquantized weights for the quantizer, fp16 [M, K]: normal with
    standard deviation sigma (drawn in float32, rounded to fp16), a fraction
    `outliers` of them scaled by 20 (the heavy tail of trained linears).
    Stream 3 of the weight seed, so it is independent of the code, scale
    and zero draws."""
    rng = np.random.default_rng([wid, layer, proj, 3])
    w = rng.standard_normal((M, K), dtype=np.float32) * np.float32(sigma)
    mask = rng.random((M, K)) < outliers
    w[mask] *= np.float32(20.0)
    return w.astype(np.float16)


def hidden_states(N, K, wid=0, layer=0, outlier_channels=0.01):
    """Inputs of the residual add + RMS normalization, token-major:
    (x fp16 [N, K], residual fp16 [N, K], gamma fp16 [K]).

    residual ~ N(0, 1) with a fixed fraction of channels 10x larger (the
    outlier channels of LLaMA hidden states), x ~ N(0, 0.5^2) (a sublayer's
    output), gamma uniform in [0.1, 1.2]; all drawn in float32 and rounded to
    fp16.  Stream 4 of (wid, layer); tokens are rows, so a prefix of N rows
    is the same for every larger N."""
    rng = np.random.default_rng([wid, layer, 0, 4])
    big = rng.random(K) < outlier_channels
    gamma = rng.uniform(0.1, 1.2, K).astype(np.float32).astype(np.float16)
    rows = np.random.default_rng([wid, layer, 1, 4])
    res = rows.standard_normal((N, 2, K), dtype=np.float32)
    residual = res[:, 0, :] * np.where(big, np.float32(10.0), np.float32(1.0))[None, :]
    x = res[:, 1, :] * np.float32(0.5)
    return x.astype(np.float16), residual.astype(np.float16), gamma


def attention_inputs(B, H, D, S, wid=0, layer=0):
    """Inputs of one decode step of attention: (qkv fp16 [B, 3 H D],
    k_cache fp16 [B, H, S, D], v_cache fp16 [B, H, S, D]), all standard
    normal (drawn in float32, rounded to fp16), so that scores q.k / sqrt(D)
    have unit spread.  Stream 5 of (wid, layer)."""
    rng = np.random.default_rng([wid, layer, 0, 5])
    qkv = rng.standard_normal((B, 3 * H * D), dtype=np.float32).astype(np.float16)
    kc = rng.standard_normal((B, H, S, D), dtype=np.float32).astype(np.float16)
    vc = rng.standard_normal((B, H, S, D), dtype=np.float32).astype(np.float16)
    return qkv, kc, vc
