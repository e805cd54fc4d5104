"""Planted mistakes in the oracle must each be caught by a pin.

Every mutant is a copy of ``oracle/pkv_oracle.c`` with one plausible mistake
(a dropped term, a wrong sign or index, a transposed operand), built with gcc
into a temporary directory and run through all pins on the CPU, in a child
process: a mutant that corrupts memory and crashes counts as caught.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "pkv_oracle.c")

MUTANTS = {
    "page_slot_swapped": ("int64_t logical_block = j / pool->page_size;\n    int64_t slot = j % pool->page_size;",
                          "int64_t logical_block = j % pool->page_size;\n    int64_t slot = j / pool->page_size;"),
    "slot_uses_head_stride": ("slot * pool->s_tok", "slot * pool->s_head"),
    "head_uses_token_stride": ("(int64_t)g * pool->s_head", "(int64_t)g * pool->s_tok"),
    "gqa_interleaved": ("int g = h / group;", "int g = h % job->pool->num_kv_heads;"),
    "causal_off_by_one": ("kv - q_len + i + 1 : kv", "kv - q_len + i : kv"),
    "causal_top_left": ("kv - q_len + i + 1 : kv", "i + 1 : kv"),
    "scale_dropped": ("scores[j] = scale * dot;", "scores[j] = dot;"),
    "exp_sign": ("double w = exp(scores[j] - m);", "double w = exp(m - scores[j]);"),
    "lse_max_dropped": ("*lse_out = m + log(z);", "*lse_out = log(z);"),
    "no_normalisation": ("out_row[d] /= z;", "out_row[d] /= 1.0;"),
    "max_wrong_way": ("if (scores[j] > m)", "if (scores[j] < m)"),
    "append_off_by_one": ("int64_t pos = (int64_t)cache_seqlens[b] + t;",
                          "int64_t pos = (int64_t)cache_seqlens[b] + t + 1;"),
    "append_source_row": ("int64_t src = ((first + t) * H + g) * (int64_t)D;",
                          "int64_t src = (first * H + g) * (int64_t)D;"),
    "append_k_into_v": ("copy_elem(v_cache, dst + d, v_new, src + d, pool->dtype);",
                        "copy_elem(v_cache, dst + d, k_new, src + d, pool->dtype);"),
    "qk_uses_v": ("load_elem(k_cache, base + d, pool->dtype);",
                  "load_elem(v_cache, base + d, pool->dtype);"),
    "bf16_widening": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "seqlens_out_not_advanced": ("seqlens_out[b] = (int32_t)(cache_seqlens[b] + n_new);",
                                 "seqlens_out[b] = (int32_t)(cache_seqlens[b]);"),
    "empty_row_lse_zero": ("*lse_out = -INFINITY;", "*lse_out = 0.0;"),
    "q_head_index": ("(token * job->num_q_heads + h) * (int64_t)D",
                     "(token * job->num_q_heads) * (int64_t)D"),
    "pair_count_dropped": ("visible > 0 ? visible : 0", "visible > 1 ? visible - 1 : 0"),
    "rope_sin_sign": ("double ra = a * ci - b * si;", "double ra = a * ci + b * si;"),
    "rope_uses_rotated_a": ("double rb = b * ci + a * si;", "double rb = b * ci + ra * si;"),
    "rope_half_pairing": ("(interleaved ? 2 * i + 1 : i + half)", "(interleaved ? 2 * i + 1 : half - 1 - i)"),
    "rope_interleaved_pairing": ("(interleaved ? 2 * i : i)", "(interleaved ? i : i)"),
    "rope_position_off_by_one": ("const float *c = cos_table + (int64_t)positions[r] * half;",
                                 "const float *c = cos_table + (int64_t)(positions[r] + 1) * half;"),
    "rope_cos_sin_swapped": ("double ci = (double)c[i], si = (double)s[i];",
                             "double ci = (double)s[i], si = (double)c[i];"),
    "rope_bf16_truncates": ("double r = ldexp(rint(ldexp(v, -qexp)), qexp);",
                            "double r = ldexp(trunc(ldexp(v, -qexp)), qexp);"),
    "rope_bf16_one_bit_short": ("int qexp = (e < -125 ? -125 : e) - 8;", "int qexp = (e < -125 ? -125 : e) - 7;"),
    "route_offset_head": ("token_offset(pool, block_table, bt_cols, b, j, 0) : -1",
                          "token_offset(pool, block_table, bt_cols, b, j, 1) : -1"),
}


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants")
    shutil.copy(os.path.join(os.path.dirname(SRC), "pkv_oracle.h"), d)
    return d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(workdir, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    path = workdir / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(str(path), str(workdir / f"lib{name}.so"))
    here = os.path.dirname(os.path.abspath(__file__))
    child = (
        "import sys\n"
        f"sys.path[:0] = [{here!r}, {os.path.dirname(here)!r}]\n"
        "import oracle\n"
        "from oracle_pins import ALL_PINS\n"
        f"orc = oracle.load({lib!r})\n"
        "caught = []\n"
        "for pin in ALL_PINS:\n"
        "    try:\n"
        "        pin(orc)\n"
        "    except Exception as e:\n"
        "        caught.append(pin.__name__)\n"
        "print('CAUGHT', caught)\n"
        "sys.exit(3 if caught else 0)\n"
    )
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin caught mutant {name}: {r.stdout[-500:]}"
