"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The copy is patched and built in a temporary directory and run in a child
process (a mutant may read out of bounds); the oracle itself is never changed.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")
HDR = os.path.join(ROOT, "oracle", "pkv_oracle.h")

# (name, original text, planted text)
MUTANTS = [
    ("interleaved_head_map", "int32_t h = kvh * group + g;",
     "int32_t h = g * w->num_kv_heads + kvh;"),
    ("dropped_scale", "scores[t] = scale * dot;", "scores[t] = dot;"),
    ("wrong_exp_sign", "scores[t] = exp(scores[t] - m);", "scores[t] = exp(m - scores[t]);"),
    ("no_max_subtraction", "scores[t] = exp(scores[t] - m);", "scores[t] = exp(scores[t]);"),
    ("exclusive_causal_diagonal", "c + i + 1, kvh", "c + i, kvh"),
    ("causal_sees_one_future", "c + i + 1, kvh", "(c + i + 2 < c + n ? c + i + 2 : c + n), kvh"),
    ("no_normalisation", "out_row[x] /= z;", "(void)z;"),
    ("offset_off_by_one", "int64_t offset = t % block_size;\n        const uint16_t *key",
     "int64_t offset = (t + 1) % block_size;\n        const uint16_t *key"),
    ("value_read_from_key_cache", "v_cache + ((block * num_kv_heads", "k_cache + ((block * num_kv_heads"),
    ("logical_block_not_translated", "int64_t block = block_table[t / block_size];\n        int64_t offset = t % block_size;\n        const uint16_t *value",
     "int64_t block = t / block_size;\n        int64_t offset = t % block_size;\n        const uint16_t *value"),
    ("store_v_from_k", "v_cache[dst] = v[src];", "v_cache[dst] = k[src];"),
    ("store_head_token_transposed",
     "int64_t dst = ((block * num_kv_heads + h) * block_size + offset) * head_dim + x;",
     "int64_t dst = ((block * block_size + offset) * num_kv_heads + h) * head_dim + x;"),
    ("store_no_skip", "if (slot < 0)\n            continue;\n        int64_t block",
     "if (slot < 0)\n            slot = 0;\n        int64_t block"),
    ("kv_bytes_without_kv_factor", "return (uint64_t)2 * (uint64_t)num_layers", "return (uint64_t)1 * (uint64_t)num_layers"),
    ("ctx_zero_not_zero", "for (int32_t x = 0; x < head_dim; ++x)\n        out_row[x] = 0.0;\n    if (n <= 0)\n        return;",
     "for (int32_t x = 0; x < head_dim; ++x)\n        out_row[x] = 0.0;\n    if (n <= 0)\n        n = 1;"),
    # FP8 cache
    ("fp8_exponent_bias_off_by_one", "v = ldexp(8.0 + (double)m, e - 10);",
     "v = ldexp(8.0 + (double)m, e - 9);"),
    ("fp8_subnormals_as_normals", "v = ldexp((double)m, -9);", "v = ldexp(8.0 + (double)m, -10);"),
    ("fp8_ties_up", "pick = ((long long)(lo / spacing) % 2 == 0) ? lo : hi;", "pick = hi;"),
    ("fp8_truncating_encode", "if (a - lo < hi - a)\n        pick = lo;",
     "if (1)\n        pick = lo;"),
    ("fp8_scale_max_240", "amax / 448.0f", "amax / 240.0f"),
    ("fp8_scale_not_applied", "* (double)scales[r];", "* 1.0;"),
    ("fp8_v_stored_from_k", "quantize_row(v + src, head_dim, v_codes", "quantize_row(k + src, head_dim, v_codes"),
    ("fp8_decode_v_from_k", "o[x] += scores[t] * vd[row * head_dim + x];",
     "o[x] += scores[t] * kd[row * head_dim + x];"),
    ("fp8_prefill_exclusive_diagonal", "attend_one_f64(q_row, w->kd, w->vd, bt, c + i + 1, kvh",
     "attend_one_f64(q_row, w->kd, w->vd, bt, c + i, kvh"),
    ("fp8_prefill_v_from_k", "out_row[x] += scores[t] * vd[row * head_dim + x];",
     "out_row[x] += scores[t] * kd[row * head_dim + x];"),
    ("fp8_prefill_key_block_untranslated",
     "int64_t row = ((int64_t)block_table[t / block_size] * num_kv_heads + kv_head) *\n                          block_size + t % block_size;\n        double dot",
     "int64_t row = ((int64_t)(t / block_size) * num_kv_heads + kv_head) *\n                          block_size + t % block_size;\n        double dot"),
    ("fp8_prefill_scale_dropped",
     "dot += bf16_bits_to_double(q_row[x]) * kd[row * head_dim + x];\n        scores[t] = scale * dot;",
     "dot += bf16_bits_to_double(q_row[x]) * kd[row * head_dim + x];\n        scores[t] = dot;"),
    # rotary position embedding
    ("rope_rotates_backwards", "float y1 = a - b;", "float y1 = a + b;"),
    ("rope_interleaved_pairs", "float x2 = bf16_bits_to_float(xr[i + half]);",
     "float x2 = bf16_bits_to_float(xr[(i + 1) % head_dim]);"),
    ("rope_cos_sin_swapped", "const float *sn = c + half;", "const float *sn = c; c = c + half;"),
    ("rope_truncates", "u += 0x7fffu + lsb;", "u += 0u * lsb;"),
    # block copy
    ("copy_direction_swapped",
     "memcpy(pools[p] + dst * block_bytes, pools[p] + src * block_bytes,",
     "memcpy(pools[p] + src * block_bytes, pools[p] + dst * block_bytes,"),
    ("copy_first_pool_only", "for (int32_t p = 0; p < num_pools; ++p)\n            memcpy",
     "for (int32_t p = 0; p < 1; ++p)\n            memcpy"),
    ("copy_order_unchecked", "rc = PKO_ERR_DUPLICATE;", "(void)0;"),
]


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, name, orig, planted):
    import oracle

    text = open(SRC).read()
    assert text.count(orig) >= 1, f"mutation site for {name} not found"
    mutated = text.replace(orig, planted, 1)
    src = tmp_path / "pkv_oracle.c"
    src.write_text(mutated)
    shutil.copy(HDR, tmp_path / "pkv_oracle.h")
    lib = tmp_path / "libmutant.so"
    oracle.build(src=str(src), out=str(lib))
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "run_pins.py"), str(lib)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr}"
