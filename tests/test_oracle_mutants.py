"""The pins must be able to fail: plant plausible mistakes in a copy of the
oracle's C source (never in the GPU path), rebuild it, and check that the pin
suite rejects every mutant."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "gate_up_swapped": ("hbuf[i] = oracle_silu(g) * u;", "hbuf[i] = oracle_silu(u) * g;"),
    "up_dropped": ("hbuf[i] = oracle_silu(g) * u;", "hbuf[i] = oracle_silu(g);"),
    "w2_transposed": ("elem(w2e, dtype, j * I + i)", "elem(w2e, dtype, (i * H + j) % (H * I))"),
    "w1_up_offset": ("(I + i) * H + h", "(i + 1) % (2 * I) * H + h"),
    "segment_reversed": ("int32_t r = offsets[e] + fill[e];", "int32_t r = offsets[e + 1] - 1 - fill[e];"),
    "expert0_dropped": ("return (e >= 0 && e < (int64_t)E) ? (int)e : -1;",
                        "return (e > 0 && e < (int64_t)E) ? (int)e : -1;"),
    "weight_index": ("hbuf, o);\n            double wk = w ? (double)w[t * K + k] : 1.0;",
                     "hbuf, o);\n            double wk = w ? (double)w[(k * T + t) % (T * K)] : 1.0;"),
    "combine_unweighted": ("double wk = w ? (double)w[t * K + k] : 1.0;\n            for (int64_t j = 0; j < H; ++j) yt[j] += wk * elem(",
                           "double wk = 1.0;\n            for (int64_t j = 0; j < H; ++j) yt[j] += wk * elem("),
    "bf16_widen": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "epilogue_stops_at_gap": ("            if (row < 0) continue;\n            for (int64_t h = 0; h < H; ++h) yt[h] += elem(recv",
                              "            if (row < 0) break;\n            for (int64_t h = 0; h < H; ++h) yt[h] += elem(recv"),
    "epilogue_first_only": ("for (int32_t j = 0; j < J; ++j) {\n            const int32_t row = src[t * J + j];",
                            "for (int32_t j = 0; j < (J > 1 ? J - 1 : J); ++j) {\n            const int32_t row = src[t * J + j];"),
    "padding_off_by_one": ("return t - j * B < (int64_t)block_counts[j];",
                           "return t - j * B <= (int64_t)block_counts[j];"),
    "padding_block_index": ("int64_t j = t / B;\n    return t - j * B", "int64_t j = t % B;\n    return t - j * B"),
    "compact_reversed": ("memcpy((char*)dst + n * row_bytes, (const char*)src + t * row_bytes",
                         "memcpy((char*)dst + (T - 1 - t) % (n + 1) * row_bytes, (const char*)src + t * row_bytes"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mut_c = tmp_path / "moe_oracle.c"
    mut_c.write_text(src.replace(old, new))
    (tmp_path / "moe_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "moe_oracle.h")).read())
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(mut_c), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
