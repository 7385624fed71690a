"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Every mutant is a copy of the whole `oracle` package with one plausible
mistake written into its source -- a dropped term, a wrong index, a
transposed operand, a wrong sign -- imported under a fresh package name.
The pins of tests/oracle_pins.py then run against it; a mutant that passes
every pin would mean the pins cannot tell that mistake from the truth.
"""

import ast
import importlib.util
import os
import shutil
import sys
import uuid

import pytest

from tests.oracle_pins import ALL_PINS

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(
    os.path.abspath(__file__))), "oracle")

MUTANTS = [
    # (id, file, original text, planted text)
    ("gqa_interleaved", "paged_attention.py",
     "for h in range(g * group, (g + 1) * group):\n                out[s, h]",
     "for h in range(g, Hq, num_kv_heads):\n                out[s, h]"),
    ("table_index_by_offset", "paged_attention.py",
     "dtype=np.int64)[t // block_size]", "dtype=np.int64)[t % block_size]"),
    ("slot_by_block", "paged_attention.py",
     "slot = t % block_size", "slot = t // block_size"),
    ("scale_dropped", "paged_attention.py",
     "logits = scale * (keys @ q)", "logits = keys @ q"),
    ("denominator_is_count", "paged_attention.py",
     "return (w @ values) / w.sum()", "return (w @ values) / len(w)"),
    ("pv_reads_keys", "paged_attention.py",
     "return (w @ values) / w.sum()", "return (w @ keys) / w.sum()"),
    ("empty_sequence_ones", "paged_attention.py",
     "return np.zeros(values.shape[1], dtype=np.float64)",
     "return np.ones(values.shape[1], dtype=np.float64)"),
    ("kv_head_ignored", "paged_attention.py",
     "cache[physical, kv_head, slot, :]", "cache[physical, 0, slot, :]"),
    ("last_token_dropped", "paged_attention.py",
     "t = np.arange(context_len)", "t = np.arange(max(context_len - 1, 0))"),
    ("query_head_is_kv_head", "paged_attention.py",
     "attention_one_head(q_s[h], keys, values, scale64)",
     "attention_one_head(q_s[g], keys, values, scale64)"),
    ("max_replaced_by_min", "paged_attention.py",
     "np.exp(logits - logits.max())", "np.exp(logits - logits.min())"),
    ("merge_sign", "paged_attention.py",
     "num = sum(s_p * np.exp(m_p - M) * o_p",
     "num = sum(s_p * np.exp(M - m_p) * o_p"),
    ("partition_short_by_one", "paged_attention.py",
     "k_p = keys[start:start + partition_size]",
     "k_p = keys[start:start + partition_size - 1]"),
    ("partial_sum_unshifted", "paged_attention.py",
     "w = np.exp(logits - m_p)", "w = np.exp(logits)"),
    ("reshape_block_offset_swapped", "cache_ops.py",
     "block, offset = divmod(int(slot), block_size)",
     "offset, block = divmod(int(slot), block_size)"),
    ("reshape_key_gets_value", "cache_ops.py",
     "kc[block, :, offset, :] = kb[i]", "kc[block, :, offset, :] = vb[i]"),
    ("reshape_writes_padding", "cache_ops.py",
     "if slot < 0:\n            continue", "if slot < -1:\n            continue"),
    ("copy_direction", "cache_ops.py",
     "kc[d] = k_src[s]", "kc[s] = k_src[d]"),
    ("copy_value_from_key", "cache_ops.py",
     "vc[d] = v_src[s]", "vc[d] = k_src[s]"),
    ("bytes_single_vector", "kv_accounting.py",
     "return 2 * hidden * layers * bytes_per_elem",
     "return hidden * layers * bytes_per_elem"),
    ("waste_off_by_one", "kv_accounting.py",
     "* block_size - context_len\n", "* block_size - context_len - 1\n"),
    ("bf16_shift", "formats.py", "<< 16", "<< 15"),
    ("e4m3_bias_8", "fp8.py", "2.0 ** (e - 7.0)", "2.0 ** (e - 8.0)"),
    ("e4m3_subnormal_scale", "fp8.py", "(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    ("e4m3_no_nan_code", "fp8.py", "mag = np.where((e == 15) & (m == 7), np.nan, mag)",
     "mag = mag"),
    ("e4m3_truncates", "fp8.py", "f8 = np.rint((2.0 * mant - 1.0) * 8.0)",
     "f8 = np.floor((2.0 * mant - 1.0) * 8.0)"),
    ("e4m3_saturates_to_nan", "fp8.py", "code = np.where(a >= MAX, 126.0, code)",
     "code = np.where(a >= MAX, 127.0, code)"),
    ("e4m3_subnormal_grid", "fp8.py", "q_sub = np.rint(a * 512.0)", "q_sub = np.rint(a * 256.0)"),
    ("e4m3_quantize_multiplies", "fp8.py", "q = v / np.float32(scale)",
     "q = v * np.float32(scale)"),
    ("fp8_key_scale_dropped", "paged_attention.py",
     "L, g, kv_dtype,\n                                      block_size) * k_scale64",
     "L, g, kv_dtype,\n                                      block_size)"),
    ("fp8_value_scale_dropped", "paged_attention.py",
     "kv_dtype, block_size) * v_scale64", "kv_dtype, block_size)"),
    ("reshape_fp8_key_scale_for_value", "cache_ops.py",
     "vq = quantize(value, dtype, v_scale)", "vq = quantize(value, dtype, k_scale)"),
    ("prefill_ignores_prefix", "prefill.py",
     "visible = L - n + i + 1", "visible = i + 1"),
    ("prefill_excludes_self", "prefill.py",
     "visible = L - n + i + 1", "visible = L - n + i"),
    ("prefill_sees_future", "prefill.py",
     "visible = L - n + i + 1", "visible = L"),
    ("prefill_rows_of_first_sequence", "prefill.py",
     "out[qsl[s] + i, h] = attention_one_head", "out[i, h] = attention_one_head"),
    ("prefill_gqa_interleaved", "prefill.py",
     "for h in range(g * group, (g + 1) * group):\n                    out[qsl[s] + i, h]",
     "for h in range(g, Hq, num_kv_heads):\n                    out[qsl[s] + i, h]"),
    ("prefill_values_are_keys", "prefill.py",
     "keys[:visible],\n                                                            values[:visible]",
     "keys[:visible],\n                                                            keys[:visible]"),
]


def _code_only(src):
    """AST of a source with every docstring removed."""
    tree = ast.parse(src)
    for node in ast.walk(tree):
        body = getattr(node, "body", None)
        if (isinstance(body, list) and body and isinstance(body[0], ast.Expr)
                and isinstance(body[0].value, ast.Constant)
                and isinstance(body[0].value.value, str)):
            node.body = body[1:] or [ast.Pass()]
    return ast.dump(tree)


def load_mutant(tmp_path, fname, old, new):
    name = "oracle_mutant_" + uuid.uuid4().hex[:8]
    dst = os.path.join(str(tmp_path), name)
    shutil.copytree(ORACLE_DIR, dst,
                    ignore=shutil.ignore_patterns("__pycache__"))
    path = os.path.join(dst, fname)
    with open(path) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site not found in {fname}: {old!r}"
    mutated = src.replace(old, new, 1)
    # the planted text must change code, not a docstring or comment
    assert _code_only(src) != _code_only(mutated), old
    with open(path, "w") as f:
        f.write(mutated)
    spec = importlib.util.spec_from_file_location(
        name, os.path.join(dst, "__init__.py"), submodule_search_locations=[dst])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("mid,fname,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mid, fname, old, new):
    mutant = load_mutant(tmp_path, fname, old, new)
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception:
            return  # caught
    pytest.fail(f"planted mistake {mid!r} passes every pin")
