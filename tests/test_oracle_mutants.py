"""Plant a mistake in a copy of the oracle (on the CPU) and check that the
pins catch it.  Each mutant is a one-line textual change of oracle.c,
compiled to a temporary library that replaces the real one for the test."""
from __future__ import annotations

import os

import pytest

import oracle
import test_oracle as T
import test_oracle_prefill as TP

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, planted text, pins that must fail)
MUTANTS = [
    ("score_sign", "x[t] = scale * dot;", "x[t] = -scale * dot;",
     ["test_hand_weights"]),
    ("no_normalisation", "double a = x[t] / Z;", "double a = x[t];",
     ["test_hand_weights", "test_weights_convex"]),
    ("exp_of_block_sum", "x[t] = exp(x[t] - m);", "x[t] = exp(x[t] - m) * (1 + (t % 2));",
     ["test_hand_weights"]),
    ("block_index_transposed", "int32_t b = row[t / B];", "int32_t b = row[t % B];",
     ["test_fig6_slots_and_gather"]),
    ("offset_transposed",
     "size_t base = pool_index(layout, (size_t)b, (size_t)(t % B), (size_t)g, B, Hkv, D);",
     "size_t base = pool_index(layout, (size_t)b, (size_t)((t / B) % B), (size_t)g, B, Hkv, D);",
     ["test_fig6_slots_and_gather", "test_hand_weights"]),
    ("head_major_swapped", "return ((b * Hkv + g) * B + o) * D;", "return ((b * B + o) * Hkv + g) * D;",
     ["test_head_major_layout_matches_transpose"]),
    ("head_map_interleaved", "int s = units ? units[2 * u] : u / Hq;\n        int h = units ? units[2 * u + 1] : u % Hq;\n        int n = context_lens[s];\n        int g = h / G;\n        size_t nn = n > 0 ? (size_t)n : 1;\n        double *K = malloc(nn * D * sizeof(double));\n        double *V = malloc(nn * D * sizeof(double));\n        double *x = malloc(nn * sizeof(double));\n        double *qv = malloc((size_t)D * sizeof(double));\n        if (!K || !V || !x || !qv) {\n            err = -1;\n        } else {\n            const int32_t",
     "int s = units ? units[2 * u] : u / Hq;\n        int h = units ? units[2 * u + 1] : u % Hq;\n        int n = context_lens[s];\n        int g = h % Hkv;\n        size_t nn = n > 0 ? (size_t)n : 1;\n        double *K = malloc(nn * D * sizeof(double));\n        double *V = malloc(nn * D * sizeof(double));\n        double *x = malloc(nn * sizeof(double));\n        double *qv = malloc((size_t)D * sizeof(double));\n        if (!K || !V || !x || !qv) {\n            err = -1;\n        } else {\n            const int32_t",
     ["test_gqa_head_map_contiguous_groups"]),
    ("half_bias", "v = ldexp((double)(f | 0x400), e - 25);", "v = ldexp((double)(f | 0x400), e - 24);",
     ["test_half_widening_exhaustive"]),
    ("merge_sign", "double cp = exp(mp - Mn);", "double cp = exp(Mn - mp);",
     ["test_split_merge_identity"]),
    ("write_offset",
     "size_t dst = pool_index(layout, (size_t)(slot / B), (size_t)(slot % B), (size_t)g,",
     "size_t dst = pool_index(layout, (size_t)(slot / B), (size_t)((slot + 1) % B), (size_t)g,",
     ["test_fig6_slots_and_gather", "test_cache_write_matches_numpy_scatter"]),
    ("copy_direction", "memmove((char *)k_cache + dst, (const char *)k_cache + src, blk);",
     "memmove((char *)k_cache + src, (const char *)k_cache + dst, blk);",
     ["test_copy_blocks_matches_numpy", "test_internals_cow_trace"]),
    ("prefill_position_off_by_one", "const int pos = len - rows + r;",
     "const int pos = len - rows + r - 1;",
     ["prefill:test_last_row_is_decode", "prefill:test_matches_numpy_masked_softmax"]),
    ("prefill_not_causal", "attend(qrow, Kc, Vc, pos + 1, D, scale, out + at, NULL, scratch);",
     "attend(qrow, Kc, Vc, len, D, scale, out + at, NULL, scratch);",
     ["prefill:test_causal_future_tokens_do_not_matter",
      "prefill:test_single_row_at_position_is_decode_of_prefix"]),
    ("prefill_wrong_kv_head", "const int kv = head / group;", "const int kv = head % Hkv;",
     ["prefill:test_matches_numpy_masked_softmax"]),
]


def _run(name, golden):
    fn = getattr(TP, name.split(":", 1)[1]) if name.startswith("prefill:") else getattr(T, name)
    import inspect

    params = inspect.signature(fn).parameters
    if "golden" in params:
        return fn(golden)
    if "dtype" in params and "P" not in params:
        for dt in ("f32", "f16", "bf16"):
            fn(dt)
        return None
    if "P" in params:
        for P in (16, 48):
            fn(P)
        return None
    return fn()


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant, tmp_path, monkeypatch, golden):
    name, old, new, pins = mutant
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(src=str(path), out=str(tmp_path / "libmutant.so")))
    monkeypatch.setattr(oracle, "_lib", lib)
    for pin in pins:
        with pytest.raises((AssertionError, oracle.OracleError)):
            _run(pin, golden)
