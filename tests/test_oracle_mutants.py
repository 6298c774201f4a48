"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks the pins catch each.

Every mutant is one textual change to oracle.c, built into a temporary library;
the test fails if all pins still pass on it.  Mutants stay inside the buffers
the pins pass, so a mutant build can only give wrong numbers, never crash.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = [
    ("scale dropped", "score[j] = dot * scale;", "score[j] = dot;"),
    ("causal off by one", "visible[j] = (j <= t)", "visible[j] = (j < t)"),
    ("mask lets in the next token", "visible[j] = (j <= t)", "visible[j] = (j <= t + 1)"),
    ("no normalisation", "score[j] = visible[j] ? score[j] / denom : 0.0;",
     "score[j] = visible[j] ? score[j] : 0.0;"),
    ("no max subtraction kept sign", "score[j] = exp(score[j] - m);",
     "score[j] = exp(m - score[j]);"),
    ("values read from the key cache", "out_row[d] += score[j] * decode(dtype, v_head",
     "out_row[d] += score[j] * decode(dtype, k_head"),
    ("interleaved head mapping", "int32_t h = hq / group;", "int32_t h = hq % Hkv;"),
    ("transposed key operand", "decode(dtype, k_head[(size_t)j * D + d])",
     "decode(dtype, k_head[(size_t)d * S + j])"),
    ("append source in head-major order",
     "size_t src = (((size_t)b * q_len + i) * Hkv + h) * D;",
     "size_t src = (((size_t)b * Hkv + h) * q_len + i) * D;"),
    ("append every draft token to the first slot", "* S + (size_t)(seq_pos[b] + i)) * D;",
     "* S + (size_t)(seq_pos[b])) * D;"),
    ("bf16 exponent bias", "ldexp(1.0 + frac / 128.0, expo - 127)",
     "ldexp(1.0 + frac / 128.0, expo - 126)"),
    ("fp16 fraction width", "ldexp(1.0 + frac / 1024.0, expo - 15)",
     "ldexp(1.0 + frac / 512.0, expo - 15)"),
    ("query token position ignored", "seq_pos[b] + i, seq_pos[b] + q_len, scale",
     "seq_pos[b], seq_pos[b] + q_len, scale"),
    ("rope rotation sign", "y[j] = encode(dtype, x1 * c - x2 * s);",
     "y[j] = encode(dtype, x1 * c + x2 * s);"),
    ("rope pairs adjacent dims", "x2 = decode(dtype, x[j + half]);", "x2 = decode(dtype, x[j ^ 1]);"),
    ("rope angle in double precision",
     "const float a = (float)((double)(float)pos[r] * (double)freqs[j]);",
     "const double a = (double)pos[r] * (double)freqs[j];"),
    ("rope position off by one", "(double)(float)pos[r] * (double)freqs[j]",
     "(double)(float)(pos[r] + 1) * (double)freqs[j]"),
    ("encode truncates", "double n = nearbyint(ax / quantum);", "double n = floor(ax / quantum);"),
    ("encode ties away from zero", "double n = nearbyint(ax / quantum);", "double n = round(ax / quantum);"),
    ("paged pool token-major inside a page",
     "const uint16_t *src = pool + (((int64_t)page * Hkv + h) * page_size + t % page_size) * D;",
     "const uint16_t *src = pool + (((int64_t)page * page_size + t % page_size) * Hkv + h) * D;"),
    ("paged block table row stride", "const int32_t page = block_table[(int64_t)b * pages_per_seq + t / page_size];\n                const uint16_t *src",
     "const int32_t page = block_table[(int64_t)b + t / page_size];\n                const uint16_t *src"),
    ("paged append into the next token", "const size_t dst = (((size_t)page * Hkv + h) * page_size + (size_t)(t % page_size)) * D;",
     "const size_t dst = (((size_t)page * Hkv + h) * page_size + (size_t)((t + 1) % page_size)) * D;"),
    ("partial rope skips a pass-through dim", "for (int32_t j = R; j < D; ++j)",
     "for (int32_t j = R + 1; j < D; ++j)"),
    ("gate sign", "out[i] *= 1.0 / (1.0 + exp(-decode(dtype, gate[i])));",
     "out[i] *= 1.0 / (1.0 + exp(decode(dtype, gate[i])));"),
    ("encode subnormal quantum", "e = emin;                   /* subnormals",
     "e = emin - 1;               /* subnormals"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation target not found once: {old!r}"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(mutant_c),
                    "-o", str(lib), "-lm"], check=True)
    orc = oracle.Oracle(str(lib))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant '{name}'"
