"""Plant plausible mistakes in a copy of the oracle, on the CPU, and check
that the pins in ``oracle_pins`` catch every one of them.

Each mutation is a textual edit of the oracle's source; the mutated source is
executed as a fresh module, and at least one pin must then fail.
"""

import inspect
import types

import pytest

import oracle.w4a16 as ora
from oracle_pins import ALL_PINS

MUTATIONS = {
    "sign_of_zero": ("((qf - zf) * sf)", "((zf - qf) * sf)"),
    "zero_not_subtracted": ("((qf - zf) * sf)", "((qf - 0 * zf) * sf)"),
    "scale_not_applied": ("((qf - zf) * sf)", "((qf - zf) * (sf * 0 + 1))"),
    "nibble_order_reversed": ("out[:, j::8] = (words >> np.uint32(4 * j))",
                              "out[:, 7 - j::8] = (words >> np.uint32(4 * j))"),
    "pack_high_nibble_first": ("words |= padded[:, j::8] << np.uint32(4 * j)",
                               "words |= padded[:, j::8] << np.uint32(28 - 4 * j)"),
    "group_of_zero_shifted": ("zf = z.astype(np.float64)[:, :, None]",
                              "zf = np.roll(z.astype(np.float64), 1, axis=1)[:, :, None]"),
    "group_of_scale_shifted": ("sf = s.astype(np.float64)[:, :, None]",
                               "sf = np.roll(s.astype(np.float64), 1, axis=1)[:, :, None]"),
    "scale_by_k_mod_g": ("qf = q.astype(np.float64).reshape(q.shape[0], G, GROUP)",
                         "qf = q.astype(np.float64).reshape(q.shape[0], GROUP, G).transpose(0, 2, 1)"),
    "last_group_dropped": ("return ((qf - zf) * sf).reshape(q.shape[0], K)",
                           "return np.concatenate([((qf - zf) * sf)[:, :-1], 0 * qf[:, -1:]], 1).reshape(q.shape[0], K)"),
    "x_reversed": ("        C[rows] = W @ Xf\n", "        C[rows] = W @ Xf[::-1]\n"),
    "abs_bound_wrong": ("        A[rows] = np.abs(W) @ Xa\n", "        A[rows] = np.abs(W @ Xf)\n"),
    "block_tail_lost": ("for r0 in range(0, M, step):", "for r0 in range(0, M - 1, step):"),
    "rows_ignored": ("        qpk, zpk, s = qpk[rows], zpk[rows], s[rows]\n",
                     "        qpk, zpk, s = qpk[rows], zpk[rows], s[::-1][rows]\n"),
    "tolerance_loose": ("return 5e-3 * np.asarray(A, dtype=np.float64) + 1e-3",
                        "return 5e-2 * np.asarray(A, dtype=np.float64) + 1e-3"),
    "nan_passes": ("n_bad = int(np.count_nonzero(~(ratio <= 1.0)))",
                   "n_bad = int(np.count_nonzero(ratio > 1.0) - np.count_nonzero(~finite))"),
    "quantizer_floor": ("q = np.clip(np.rint(w / s32[:, :, None])", "q = np.clip(np.floor(w / s32[:, :, None])"),
    "quantizer_zero_range": ("lo = np.minimum(w.min(axis=2), np.float32(0.0))", "lo = w.min(axis=2)"),
    "quantizer_scale_16": ("s16 = (rng / np.float32(15.0))", "s16 = (rng / np.float32(16.0))"),
    "group_size_64": ("GROUP = 128", "GROUP = 64"),
    "norm_sum_not_mean": ("ms = np.mean(h * h, axis=1)", "ms = np.sum(h * h, axis=1)"),
    "norm_mean_over_tokens": ("ms = np.mean(h * h, axis=1)", "ms = np.mean(h * h, axis=0)[:h.shape[0]]"),
    "norm_no_sqrt": ("h / np.sqrt(ms + float(eps))[:, None]", "h / (ms + float(eps))[:, None]"),
    "norm_eps_outside_sqrt": ("h / np.sqrt(ms + float(eps))[:, None]", "h / (np.sqrt(ms) + float(eps))[:, None]"),
    "norm_gain_dropped": ("* np.asarray(gamma, dtype=np.float64)[None, :]", "* 1.0"),
    "norm_gain_reversed": ("* np.asarray(gamma, dtype=np.float64)[None, :]",
                           "* np.asarray(gamma, dtype=np.float64)[None, ::-1]"),
    "norm_residual_subtracted": ("h = np.asarray(x, dtype=np.float64) + np.asarray(r, dtype=np.float64)",
                                 "h = np.asarray(x, dtype=np.float64) - np.asarray(r, dtype=np.float64)"),
    "norm_mean_subtracted": ("ms = np.mean(h * h, axis=1)",
                             "h = h - h.mean(axis=1, keepdims=True)\n    ms = np.mean(h * h, axis=1)"),
    "residual_not_rounded": ("+ np.asarray(r, dtype=np.float64)).astype(np.float16)",
                             "+ np.asarray(r, dtype=np.float64))"),
    "norm_tolerance_loose": ("return 2e-3 * np.abs(", "return 2e-1 * np.abs("),
    "rope_sin_sign": ("out[..., 0::2] = x0 * c - x1 * s", "out[..., 0::2] = x0 * c + x1 * s"),
    "rope_half_split_pairs": ("x0, x1 = x[..., 0::2], x[..., 1::2]", "x0, x1 = x[..., :D // 2], x[..., D // 2:]"),
    "rope_frequency_exponent": ("theta = float(base) ** (-2.0 * i / D)", "theta = float(base) ** (-1.0 * i / D)"),
    "rope_query_position_shifted": ("qr = rope(q, p, base)", "qr = rope(q, p + 1, base)"),
    "rope_key_not_rotated": ("kr = rope(k, p, base)", "kr = rope(k, 0, base)"),
    "attention_cache_shifted": ("Kc = np.asarray(k_cache[b, :, :p], dtype=np.float64)",
                                "Kc = np.asarray(k_cache[b, :, 1:p + 1], dtype=np.float64)"),
    "attention_new_value_dropped": ("Vall = np.concatenate([Vc, v.astype(np.float16)",
                                    "Vall = np.concatenate([Vc, 0 * v.astype(np.float16)"),
    "attention_scale_1_over_d": ("scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D"),
    "attention_bound_wrong": ("A[b, h * D:(h + 1) * D] = w @ np.abs(Vall[h])",
                              "A[b, h * D:(h + 1) * D] = np.abs(w @ Vall[h])"),
    "attention_head_slices_swapped": ("q = qkv[b, 0:H * D].reshape(H, D)", "q = qkv[b, H * D:2 * H * D].reshape(H, D)"),
    "rope_tolerance_loose": ("return 2.0 ** -11 * np.abs(ref)", "return 2.0 ** -5 * np.abs(ref)"),
    "silu_sigmoid_sign": ("return g / (1.0 + np.exp(-g)) * u", "return g / (1.0 + np.exp(g)) * u"),
    "silu_halves_swapped": ("g, u = gu[:, :I], gu[:, I:]", "u, g = gu[:, :I], gu[:, I:]"),
    "silu_no_gate": ("return g / (1.0 + np.exp(-g)) * u", "return 1.0 / (1.0 + np.exp(-g)) * u"),
    "silu_tolerance_loose": ("return 1e-3 * np.abs(np.asarray(ref", "return 1e-1 * np.abs(np.asarray(ref"),
}


def _mutant(old, new):
    src = inspect.getsource(ora)
    assert src.count(old) == 1, "mutation anchor must occur once: %r" % old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes():
    mod = _mutant("GROUP = 128", "GROUP = 128")
    for pin in ALL_PINS:
        pin(mod)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:
            caught.append(pin.__name__)
    assert caught, "no pin catches mutation %s" % name
