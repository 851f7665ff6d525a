"""Plant plausible mistakes in copies of the oracle source and show the pins catch each one.

Each mutant is a textual edit of ``oracle/w4a16_oracle.c`` compiled into a
temporary directory and exercised in a child process (a mutant may read out of
bounds, so it must not take the test runner down with it).  The product
library is never involved.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "w4a16_oracle.c")

MUTANTS = {
    "zero point 7": ("(float)(q - 8)", "(float)(q - 7)"),
    "nibble mask drops a bit": ("int q = (int)(code & 0x0F);", "int q = (int)(code & 0x07);"),
    "group of 16 in dequant": ("scales[(size_t)n * G + k / 32]", "scales[(size_t)n * G + k / 16 % G]"),
    "group of 64 in gemm": ("sw + (size_t)n * G + k / 32);\n                acc = acc + prod;",
                            "sw + (size_t)n * G + k / 64);\n                acc = acc + prod;"),
    "ties away from zero": ("(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)"),
    "truncating bf16": ("if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;", ""),
    "dropped last k": ("for (int k = 0; k < K; ++k) {\n                float prod",
                       "for (int k = 0; k < K - 1; ++k) {\n                float prod"),
    "wrong A row": ("j->A + (size_t)(i / j->a_row_div) * K", "j->A + (size_t)(i % j->a_row_div) * K"),
    "transposed weight index": ("float prod = orc_bf16_to_f32(a[k]) *\n                             orc_weight(j->fmt, cw, j->scales, (size_t)n * K + k,",
                                "float prod = orc_bf16_to_f32(a[k]) *\n                             orc_weight(j->fmt, cw, j->scales, (size_t)(k % N) * K + (n % K),"),
    "sentinel R-1": ("for (int p = 0; p < maxP; ++p) sorted_ids[p] = R;", "for (int p = 0; p < maxP; ++p) sorted_ids[p] = R - 1;"),
    "no per-expert padding": ("int padded = (cnt[e] + BM - 1) / BM * BM;", "int padded = cnt[e];"),
    "non-local id kept": ("if (e >= 0 && e < E) cnt[e] += 1;", "if (e >= 0 && e <= E) cnt[e < E ? e : 0] += 1;"),
    "silu sign": ("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    "gate and up swapped": ("h[c] = orc_silu_mul_one(gu[c], gu[I + c]);", "h[c] = orc_silu_mul_one(gu[I + c], gu[c]);"),
    "combine keeps non-local": ("                if (e < 0 || e >= E) continue;\n                acc = acc + tw",
                                "                acc = acc + tw"),
    "combine weight index": ("acc = acc + tw[(size_t)t * k + j] *", "acc = acc + tw[(size_t)t * k] *"),
    "down uses unrounded h": ("acc = acc + orc_bf16_to_f32(h[kk]) * orc_weight(j->fmt, cw, j->s2, (size_t)kk, sw + kk / 32);",
                              "acc = acc + (float)(orc_silu(gu[kk]) * gu[I + kk]) * orc_weight(j->fmt, cw, j->s2, (size_t)kk, sw + kk / 32);"),
    "e2m1 3 and 4 swapped": ("{0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f}", "{0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 4.0f, 3.0f, 6.0f}"),
    "e2m1 sign ignored": ("return (code & 8) ? -v : v;", "return v;"),
    "e8m0 bias 128": ("ldexpf(1.0f, (int)e - 127)", "ldexpf(1.0f, (int)e - 128)"),
    "mxfp4 scale of the next group": ("srow[k / 32]", "srow[(k / 32 + 1) % G]"),
    "mxfp4 scales read as bf16": ("if (fmt == 1) return orc_dequant_mxfp4_one", "if (fmt == 2) return orc_dequant_mxfp4_one"),
}

RUNNER = textwrap.dedent("""
    import sys, traceback
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    import oracle, oracle_pins
    o = oracle.Oracle({lib!r})
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except Exception as exc:  # AssertionError or a crash inside the pin
            failed.append(pin.__name__)
    print("FAILED_PINS", ",".join(failed))
""")


def test_mutation_anchors_present():
    src = open(SRC).read()
    for name, (old, _) in MUTANTS.items():
        assert old in src, name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, "mutation anchor missing: " + name
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    sys.path.insert(0, ROOT)
    import oracle

    lib = oracle.compile_oracle(str(csrc), str(tmp_path / "libmutant.so"))
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    line = [l for l in proc.stdout.splitlines() if l.startswith("FAILED_PINS")]
    caught = proc.returncode != 0 or (line and line[0].split(" ", 1)[1].strip() != "")
    assert caught, "mutant '%s' passed every pin" % name
