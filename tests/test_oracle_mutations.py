"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a *copy* of the oracle source, builds
it into a temporary library, and requires at least one pin to fail against it.
A pin set that lets a mutation through is too weak to trust the oracle with.
(The pages use the same technique on their kernels: vLLM PR #62589, Validation,
shifts the visible bound by one column on purpose; ROCm/aiter PR #4221,
curated-matrix commit, plants eleven kernel bugs.)
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTATIONS = {
    "no_relu": ("double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    "abs_not_relu": ("double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot > 0.0 ? dot : -dot;"),
    "relu_after_sum": ("acc += wh * relu;", "acc += wh * dot; if (h == num_heads - 1) acc = acc > 0.0 ? acc : 0.0;"),
    "last_head_only": ("acc += wh * relu;", "acc = wh * relu;"),
    "weights_ignored": ("double wh = w ? (double)w[(int64_t)row * num_heads + h] : 1.0;", "double wh = 1.0;"),
    "weight_index": ("w[(int64_t)row * num_heads + h]", "w[(int64_t)row * num_heads]"),
    "slot_off_by_one": ("int slot = col % block_size;", "int slot = (col + 1) % block_size;"),
    "block_index": ("block_table[(int64_t)req * max_blocks + col / block_size]",
                    "block_table[(int64_t)req * max_blocks + (col / block_size + 1) % max_blocks]"),
    "request_blind": ("int req = row_to_req[row];", "int req = row % num_reqs;"),
    "q_transposed": ("int64_t at = ((int64_t)row * num_heads + h) * head_dim + d;",
                     "int64_t at = ((int64_t)row * num_heads + d % num_heads) * head_dim + h;"),
    "ctx_minus_one": ("int64_t ctx = ctx_lens[row];\n        if (ctx < 0)\n            ctx = 0;\n        if (ctx > cap)",
                      "int64_t ctx = ctx_lens[row] - 1;\n        if (ctx < 0)\n            ctx = 0;\n        if (ctx > cap)"),
    "no_width_clamp": ("if (cap > width)\n        cap = width;", ""),
    "tail_zero": ("o[col] = -INFINITY;", "o[col] = 0.0;"),
    "scale_dropped": ("kd[d] = ora_e4m3fn_to_double(k[d]) * s;", "kd[d] = ora_e4m3fn_to_double(k[d]);"),
    "copack_scale_slot": ("4 * slot, sizeof sf);", "4 * (slot ^ 1), sizeof sf);"),
    "copack_key_stride": ("k = base + (int64_t)slot * head_dim;", "k = base + (int64_t)slot * (head_dim + 4);"),
    "fp8_bias": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "fp8_subnormal": ("v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    "fp8_no_nan": ("if (e == 15 && m == 7)\n        return NAN;", ""),
    "bf16_shift": ("uint32_t u = ((uint32_t)bits) << 16;", "uint32_t u = ((uint32_t)bits) << 15;"),
    "shuffle_transposed": ("g[(d / 16) * 256 + (slot % 16) * 16 + d % 16]", "g[(d / 16) * 16 + (slot % 16) * 256 + d % 16]"),
    "shuffle_as_flat": ("g[(d / 16) * 256 + (slot % 16) * 16 + d % 16]", "g[(slot % 16) * head_dim + d]"),
    "fp16_bias": ("v = ldexp(1.0 + (double)m / 1024.0, e - 15);", "v = ldexp(1.0 + (double)m / 1024.0, e - 14);"),
    "fp16_subnormal": ("v = ldexp((double)m / 1024.0, -14);", "v = ldexp((double)m / 1024.0, -15);"),
    "fp16_as_bf16": ("return dtype == 0 ? ora_bf16_to_double(b) : ora_fp16_to_double(b);",
                     "return ora_bf16_to_double(b);"),
    "topk_tie_reversed": ("return (a->i > b->i) - (a->i < b->i);", "return (a->i < b->i) - (a->i > b->i);"),
    "topk_ascending": ("if (a->v > b->v)\n        return -1;", "if (a->v < b->v)\n        return -1;"),
    "topk_reads_width": ("int64_t n = ctx_lens[row];", "int64_t n = width;"),
    "topk_pad_zero": ("for (int64_t j = take; j < k; ++j)\n            o[j] = -1;",
                      "for (int64_t j = take; j < k; ++j)\n            o[j] = 0;"),
    "topk_ctx_plus_one": ("int64_t n = ctx_lens[row];", "int64_t n = ctx_lens[row] + 1;"),
    "topk_nan_accepted": ("if (isnan(x[j]))\n                bad = 1;", ""),
    "topk_starts_ignored": ("int64_t s = row_starts ? row_starts[row] : 0;", "int64_t s = 0;"),
    "topk_absolute_index": ("c[j].i = (int32_t)j;", "c[j].i = (int32_t)(j + s);"),
    "topk_start_off_by_one": ("const float *x = logits + (int64_t)row * stride + s;",
                              "const float *x = logits + (int64_t)row * stride + (s > 0 ? s - 1 : 0);"),
    "expand_no_bound": ("(!token_lens || tok < (int64_t)token_lens[row]);", "1;"),
    "expand_token_offset": ("int64_t tok = (int64_t)c * ratio + j;", "int64_t tok = (int64_t)c * ratio + j + 1;"),
    "expand_keeps_padding": ("int keep = c >= 0 &&", "int keep = c >= -1 &&"),
    "expand_bound_inclusive": ("tok < (int64_t)token_lens[row]", "tok <= (int64_t)token_lens[row]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "qsa_oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / f"lib_{name}.so")
    oracle.build_lib(src=str(mutated), out=so)
    lib = oracle.load(so)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"mutation {name} survived every pin"


def test_unmutated_source_passes_all_pins(tmp_path):
    so = str(tmp_path / "lib_clean.so")
    oracle.build_lib(out=so)
    lib = oracle.load(so)
    for pin in ALL_PINS:
        pin(lib)
    assert os.path.exists(so)
