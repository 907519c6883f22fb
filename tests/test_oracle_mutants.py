"""The pins catch plausible mistakes in the oracle.

Each case copies oracle.c, plants one mistake by a textual substitution
(a dropped term, a wrong sign, a wrong index, swapped operands, a wrong
exponent bias), builds the copy with gcc in a temporary directory and runs
every pin against it: at least one pin must fail.  Nothing here touches the
committed oracle or a GPU.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    # query head -> kv head grouping taken as interleaved instead of contiguous
    "gqa_interleaved": ("int h = hq / group;", "int h = hq % a->num_kv_heads;"),
    # block-table column taken from the offset
    "table_index": ("[(int64_t)b * a->max_blocks_per_seq + t / a->block_size]",
                    "[(int64_t)b * a->max_blocks_per_seq + t % a->max_blocks_per_seq]"),
    # wrong in-block offset in the gather
    "kv_offset": ("    int off = (int)(t % a->block_size);\n    if (a->k_codes)",
                  "    int off = (int)((t + 1) % a->block_size);\n    if (a->k_codes)"),
    # head and offset swapped in the pool index
    "pool_index_order": ("((block * a->num_kv_heads + h) * a->block_size + off)",
                         "((block * a->block_size + off) * a->num_kv_heads + h)"),
    "scale_dropped": ("s[t - t0] = a->scale * dot;", "s[t - t0] = dot;"),
    "max_sign": ("s[i] = exp(s[i] - m);", "s[i] = exp(m - s[i]);"),
    "values_from_k": ("is_value ? a->v_cache : a->k_cache", "is_value ? a->k_cache : a->k_cache"),
    "no_normalisation": ("o[d] = acc / l;", "o[d] = acc;"),
    "last_dim_dropped": ("for (int d = 0; d < a->head_dim; ++d)\n            dot +=",
                         "for (int d = 0; d < a->head_dim - 1; ++d)\n            dot +="),
    "one_token_short": ("logits(a, b, hq, h, 0, L, s);\n        softmax_v(a, b, h, 0, L,",
                        "logits(a, b, hq, h, 0, L - 1, s);\n        softmax_v(a, b, h, 0, L - 1,"),
    "f16_bias": ("expo - 25", "expo - 24"),
    "f16_subnormal": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "bf16_bias": ("expo - 134", "expo - 133"),
    "split_weight": ("acc += pl[j] * exp(pm[j] - M) * po", "acc += pl[j] * po"),
    "write_offset": ("int64_t blk = s / block_size, off = s % block_size;",
                     "int64_t blk = s / block_size, off = (s + 1) % block_size;"),
    "write_v_from_k": ("(const char *)v + ((int64_t)i * v_token_stride",
                       "(const char *)k + ((int64_t)i * k_token_stride"),
    "append_position": ("if (app && t == (int64_t)a->context_lens[b] - 1)",
                        "if (app && t == (int64_t)a->context_lens[b] - 2)"),
    "write_token_stride": ("(const char *)k + ((int64_t)i * k_token_stride + (int64_t)h * head_dim)",
                           "(const char *)k + ((int64_t)i * num_kv_heads * head_dim + (int64_t)h * head_dim)"),
    # multi-token: the query's own position excluded from its keys
    "prefill_diagonal": ("    int64_t n = p + 1;\n", "    int64_t n = p;\n"),
    # multi-token: causal mask aligned to the start instead of the end of the cache
    "prefill_alignment": ("int64_t p = (int64_t)a->context_lens[b] - T + i;",
                          "int64_t p = i;"),
    # multi-token: the query row taken from the sequence index
    "prefill_query_row": ("int64_t qbase = (r * a->num_q_heads + hq)",
                          "int64_t qbase = ((int64_t)b * a->num_q_heads + hq)"),
    # multi-token: query heads interleaved over kv heads
    "prefill_gqa": ("int kvh = hq / (a->num_q_heads / a->num_kv_heads);",
                    "int kvh = hq % a->num_kv_heads;"),
    # multi-token: a row on a sequence boundary given to the previous sequence
    "prefill_sequence_search": ("while (query_start[b + 1] <= r)",
                                "while (query_start[b + 1] < r)"),
    # block copy: V taken from the K snapshot
    "copy_v_from_k": ("memcpy((char *)v_cache + dst * block_bytes, vs + src * block_bytes",
                      "memcpy((char *)v_cache + dst * block_bytes, ks + src * block_bytes"),
    # block copy: sources read from the live pools (a chain copies twice)
    "copy_no_snapshot": ("memcpy((char *)k_cache + dst * block_bytes, ks + src * block_bytes",
                         "memcpy((char *)k_cache + dst * block_bytes, (char *)k_cache + src * block_bytes"),
    # gather: the K half of a packed row taken from the V pool
    "gather_k_from_v": ("memcpy(row, (const char *)k_cache + id * block_bytes",
                        "memcpy(row, (const char *)v_cache + id * block_bytes"),
    # scatter: K restored from the V half of the packed row
    "scatter_k_offset": ("memcpy((char *)k_cache + id * block_bytes, row, ",
                         "memcpy((char *)k_cache + id * block_bytes, row + block_bytes, "),
    # rotary embedding: rotation in the wrong direction
    "rope_sign": ("y[j] = a - b;", "y[j] = a + b;"),
    # rotary embedding: pairs (j, j + 1) instead of (j, j + R/2)
    "rope_pairing": ("float a = x[j] * c, b = x[j + half] * sn;",
                     "float a = x[j] * c, b = x[j + 1] * sn;"),
    # rotary embedding: sine read from the cosine half of the table
    "rope_table_offset": ("float c = cs[j], sn = cs[half + j];", "float c = cs[j], sn = cs[j];"),
    # fp16 rounding truncates (normal binades)
    "f16_round_trunc": ("double q = rint(a / ldexp(1.0, expo - 10));",
                        "double q = floor(a / ldexp(1.0, expo - 10));"),
    # fp16 rounding truncates (subnormals)
    "f16_subnormal_trunc": ("double q = rint(a / ldexp(1.0, -24));",
                            "double q = floor(a / ldexp(1.0, -24));"),
    # bf16 rounding truncates
    "bf16_round_trunc": ("double q = rint(a / ldexp(1.0, expo - 7));",
                         "double q = floor(a / ldexp(1.0, expo - 7));"),
    # INT8: V codes stored and read in a plain token-major order
    "int8_v_token_major": ("    int jv = row / 4;\n    return base + (",
                           "    int jv = row / 4;\n    return base + (int64_t)off * a->head_dim + d + 0 * ("),
    # INT8: K code lanes of one tile swapped (row and dim group transposed)
    "int8_k_lane_order": ("16 * jk + row) * (a->head_dim / 32)", "4 * row + jk) * (a->head_dim / 32)"),
    # INT8: scale group taken modulo the group count instead of d / group_size
    "int8_scale_group": ("d / a->group_size)];", "d % (a->head_dim / a->group_size))];"),
    # INT8: K values scaled by the V scales
    "int8_k_scale_from_v": ("const float *scales = is_value ? a->v_scales : a->k_scales;",
                            "const float *scales = is_value ? a->v_scales : a->v_scales;"),
    # INT8: halfway quotients rounded away from zero
    "int8_round_half_away": ("rintf(x[i] / s)", "roundf(x[i] / s)"),
    # INT8: scale amax / 128 (code 127 never reached)
    "int8_scale_128": ("float s = amax / 127.0f;", "float s = amax / 128.0f;"),
    # INT8: codes read as unsigned bytes (two's complement sign dropped)
    "int8_code_sign": ("double c = (double)codes[", "double c = (double)(uint8_t)codes["),
    # the decode's logits take the magnitude of the scale (its sign dropped)
    "scale_sign_dropped": ("        s[t - t0] = a->scale * dot;", "        s[t - t0] = fabs(a->scale) * dot;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(path), "-lm"], check=True)
    h = oracle.lib(str(so))
    failed = []
    for pin_name, pin in oracle_pins.PINS.items():
        try:
            pin(h)
        except (AssertionError, oracle.OracleError, ValueError, FloatingPointError):
            failed.append(pin_name)
    assert failed, f"no pin caught mutant {name}"
