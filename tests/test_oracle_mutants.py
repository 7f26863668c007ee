"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is the oracle's source with one plausible slip (a wrong index,
a dropped term, a wrong rounding), executed into a fresh module on the CPU.
"""
import inspect
import types

import pytest

import oracle.paged_attention as O
from oracle_pins import ALL_PINS

SRC = inspect.getsource(O)

MUTANTS = [
    ("gqa_map_modulo_decode", "            g = h // G\n            s = sc * (K[:, g, :] @ q[b, h])",
     "            g = h % cache.num_kv_heads\n            s = sc * (K[:, g, :] @ q[b, h])"),
    ("gqa_map_modulo_prefill", "            g = h // G\n            s = np.where(seen, sc * (q[r0:r1",
     "            g = h % cache.num_kv_heads\n            s = np.where(seen, sc * (q[r0:r1"),
    ("dropped_scale", "s = sc * (K[:, g, :] @ q[b, h])", "s = (K[:, g, :] @ q[b, h])"),
    ("causal_strict", "keypos <= rowpos", "keypos < rowpos"),
    ("causal_top_left", "rowpos = P + np.arange(C)[:, None]", "rowpos = np.arange(C)[:, None]"),
    ("excludes_current_token", "n = int(context_lens[b])\n        if n == 0:",
     "n = int(context_lens[b]) - 1\n        if n <= 0:"),
    ("wrong_normalisation", "return e / np.sum(e, axis=-1, keepdims=True)",
     "return e / np.max(e, axis=-1, keepdims=True)"),
    ("page_index_off", "page = np.asarray(block_row, dtype=np.int64)[t // PAGE_SIZE]",
     "page = np.asarray(block_row, dtype=np.int64)[(t + 1) // PAGE_SIZE]"),
    ("v_layout_not_transposed", "V = upcast(cache.v[page, :, :, off], cache.dtype, vs)",
     "V = upcast(cache.v.reshape(cache.v.shape[0], cache.v.shape[1], PAGE_SIZE, -1)[page, :, off, :], cache.dtype, vs)"),
    ("swapped_int8_scales", "cache.k_scales[page, :, off] = ks", "cache.k_scales[page, :, off] = vs"),
    ("int8_scale_128", "(absmax / np.float32(127.0))", "(absmax / np.float32(128.0))"),
    ("int8_truncates", "np.clip(np.rint(ratio), -127, 127)", "np.clip(np.trunc(ratio), -127, 127)"),
    ("int8_dequant_divides", "np.asarray(stored, dtype=np.int8).astype(np.float64) * \\",
     "np.asarray(stored, dtype=np.int8).astype(np.float64) / \\"),
    ("bf16_round_half_up", "(u + 0x7FFF + ((u >> 16) & 1)) >> 16", "(u + 0x8000) >> 16"),
    ("bf16_truncates", "(u + 0x7FFF + ((u >> 16) & 1)) >> 16", "u >> 16"),
    ("append_ignores_padding", "keep = slots >= 0", "keep = slots >= -1"),
    ("window_decode_one_short", "lo = max(0, n - window) if window > 0 else 0",
     "lo = max(0, n - window + 1) if window > 0 else 0"),
    ("window_decode_one_long", "lo = max(0, n - window) if window > 0 else 0",
     "lo = max(0, n - window - 1) if window > 0 else 0"),
    ("window_prefill_mask_inclusive", "keypos > rowpos - window", "keypos >= rowpos - window"),
    ("window_prefill_from_chunk_end", "keypos > rowpos - window", "keypos > P + C - 1 - window"),
    ("window_prefill_mask_dropped", "        if window > 0:\n            seen = seen &",
     "        if window < 0:\n            seen = seen &"),
    ("prefill_unseen_v_leaks", "            if np.all(np.isfinite(Vg)):", "            if True:"),
    ("window_prefill_first_key_late", "lo = max(0, P - window + 1) if window > 0 else 0",
     "lo = max(0, P - window + 2) if window > 0 else 0"),
    ("fp8_scale_240", "(absmax / np.float32(E4M3_MAX))", "(absmax / np.float32(240.0))"),
    ("fp8_truncates", "q = np.minimum(np.rint(a / step) * step, E4M3_MAX)",
     "q = np.minimum(np.floor(a / step) * step, E4M3_MAX)"),
    ("fp8_bias_8", "bits = np.where(normal, ((qe + 7) << 3) + mant_normal, q / 2.0 ** -9)",
     "bits = np.where(normal, ((qe + 8) << 3) + mant_normal, q / 2.0 ** -9)"),
    ("fp8_subnormal_grid", "e = np.maximum(ex - 1, -6)", "e = np.maximum(ex - 1, -7)"),
    ("fp8_two_mantissa_bits", "step = np.ldexp(1.0, e - 3)", "step = np.ldexp(1.0, e - 2)"),
    ("fp8_dequant_unscaled", "return e4m3_bits_to_f64(stored) * np.asarray(scales, dtype=np.float32).astype(np.float64)",
     "return e4m3_bits_to_f64(stored)"),
    ("rope_turns_backwards", "ra = a * c - b * s\n    rb = b * c + a * s",
     "ra = a * c + b * s\n    rb = b * c - a * s"),
    ("rope_not_a_rotation", "rb = b * c + a * s", "rb = b * c - a * s"),
    ("rope_frequency_exponent", "(-2.0 * i / d)", "(-1.0 * i / d)"),
    ("rope_frequency_from_d_minus_2", "(-2.0 * i / d)", "(-2.0 * i / (d - 2))"),
    ("rope_half_reads_interleaved", "a, b = x[..., :h], x[..., h:]", "a, b = x[..., 0::2], x[..., 1::2]"),
    ("rope_position_off_by_one", "np.asarray(positions, dtype=np.float64)[:, None]",
     "(np.asarray(positions, dtype=np.float64)[:, None] + 1)"),
    ("rope_rotates_v", "ref_append(cache, k_rot.astype(np.float32), v_new, slot_mapping)",
     "ref_append(cache, k_rot.astype(np.float32), rope_f64(np.asarray(v_new, dtype=np.float32), "
     "positions, theta, style).astype(np.float32), slot_mapping)"),
    ("rope_q_left_unrotated", "return storage_from_f32(rot.astype(np.float32), dtype)",
     "return storage_from_f32(np.asarray(q, dtype=np.float32), dtype)"),
    ("rope_frequency_half_precision", ".astype(np.float32).astype(np.float64)\n    ang",
     ".astype(np.float16).astype(np.float64)\n    ang"),
    ("comparator_signed", "return float(np.max(np.abs(g - r)))", "return float(np.max(g - r))"),
    ("comparator_mean", "return float(np.max(np.abs(g - r)))", "return float(np.mean(np.abs(g - r)))"),
    ("comparator_fp32", "return float(np.max(np.abs(g - r)))",
     "return float(np.max(np.abs(g.astype(np.float32) - r.astype(np.float32))))"),
    ("comparator_gpu_only_finite", "np.all(np.isfinite(g)) and np.all(np.isfinite(r))",
     "np.all(np.isfinite(g))"),
    ("comparator_ignores_nan", "np.all(np.isfinite(g)) and np.all(np.isfinite(r))",
     "not np.any(np.isinf(g)) and not np.any(np.isinf(r))"),
    ("comparator_broadcasts", "    if g.shape != r.shape:\n        raise",
     "    if g.ndim != r.ndim and False:\n        raise"),
    ("rope_f16_intermediate", "ref_append(cache, k_rot.astype(np.float32), v_new, slot_mapping)",
     "ref_append(cache, k_rot.astype(np.float16).astype(np.float32), v_new, slot_mapping)"),
]


def _mutant_module(old, new):
    assert SRC.count(old) == 1, f"mutation target must occur once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _mutant_module(old, new)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:        # an assertion or a crash both count as caught
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
