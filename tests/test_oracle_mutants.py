"""Strength of the oracle's pins, shown rather than claimed: each case below
plants one plausible mistake in a copy of oracle/oracle.c (a wrong rounding
rule, a dropped term, a wrong sign, index or exponent bias, an off-by-one
window), builds it, and runs the pin tests of the function it touches
against that copy.  Every mutant must compile and must make its pins fail
(pytest's "tests failed" status, not a collection or build error).  The
mutants live only in a temporary directory; the real oracle is untouched."""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, exact snippet of oracle.c, its replacement, pin file that must fail)
MUTANTS = [
    ("encode rounds ties away from zero",
     "double n = nearbyint(a / quantum);", "double n = round(a / quantum);",
     "test_oracle_codec.py"),
    ("encode codes overflow as NaN instead of saturating",
     "if (a >= maxval) return sign | orc_max_code(fmt);",
     "if (a >= maxval) return sign | 0x7F;", "test_oracle_codec.py"),
    ("E5M2 exponent bias 16",
     "f->bias = 15; return 0;", "f->bias = 16; return 0;", "test_oracle_codec.py"),
    ("amax keeps the sign bit",
     "return orc_f32_bits(x) & 0x7FFFFFFFu; }", "return orc_f32_bits(x) & 0xFFFFFFFFu; }",
     "test_oracle_amax_scale.py"),
    ("cast writes the transpose row-major",
     "if (qt) qt[c * rows + r] = code;", "if (qt) qt[r * cols + c] = code;",
     "test_oracle_amax_scale.py"),
    ("scale update applies the margin with the wrong sign",
     "float denom = ldexpf(m, margin);", "float denom = ldexpf(m, -margin);",
     "test_oracle_amax_scale.py"),
    ("scale update forgets the oldest of the 16 amaxes",
     "for (int i = 1; i < H; ++i) {\n            uint32_t k = orc_abs_key(h[i]);",
     "for (int i = 1; i < H - 1; ++i) {\n            uint32_t k = orc_abs_key(h[i]);",
     "test_oracle_amax_scale.py"),
    ("scale-inverse not inverted",
     "scale_inv[t] = 1.0f / scale[t];", "scale_inv[t] = scale[t];",
     "test_oracle_amax_scale.py"),
    ("product drops the last K position",
     "for (int64_t k = 0; k < K; ++k) acc += a[k] * b[k];",
     "for (int64_t k = 0; k + 1 < K; ++k) acc += a[k] * b[k];", "test_oracle_gemm.py"),
    ("product applies the first scale-inverse twice",
     "double y = acc * (double)sinv_a * (double)sinv_b + orc_bias_at(bias, j);",
     "double y = acc * (double)sinv_a * (double)sinv_a + orc_bias_at(bias, j);",
     "test_oracle_gemm.py"),
    ("product drops the bias",
     "double y = acc * (double)sinv_a * (double)sinv_b + orc_bias_at(bias, j);",
     "double y = acc * (double)sinv_a * (double)sinv_b;", "test_oracle_gemm_fp8out.py"),
    ("bias gradient skips the last row",
     "for (int64_t r = 0; r < rows; ++r) acc += (double)orc_load_src(x, src, r * ld + c);",
     "for (int64_t r = 0; r + 1 < rows; ++r) acc += (double)orc_load_src(x, src, r * ld + c);",
     "test_oracle_dbias.py"),
    ("two-term residual add rounded once",
     "float t = orc_bf16_to_f32(orc_f32_to_bf16_canon(xv + av));", "float t = xv + av;",
     "test_oracle_produce.py"),
    ("modulation divides before multiplying",
     "out = orc_f32_to_bf16_canon(prod / bv);", "out = orc_f32_to_bf16_canon(av * (xv / bv));",
     "test_oracle_produce.py"),
    ("modulation gradient of the divisor with the wrong sign",
     "uint16_t ob = orc_f32_to_bf16_canon(-tu);", "uint16_t ob = orc_f32_to_bf16_canon(tu);",
     "test_oracle_modulate_backward.py"),
    ("dynamic scaling ignores the margin",
     "float s = fp8_max / ldexpf(amax, margin);", "float s = fp8_max / amax;",
     "test_oracle_dynamic.py"),
    ("FP8-output product casts with twice the output scale",
     "rc = orc_cast_transpose_amax(v, 1, M, N, N, scale_out, fo, q, NULL, amax_inout,",
     "rc = orc_cast_transpose_amax(v, 1, M, N, N, 2.0f * scale_out, fo, q, NULL, amax_inout,",
     "test_oracle_gemm_fp8out.py"),
]


def _run_mutant(base: str, idx: int, snippet: str, repl: str, pin: str):
    src = open(SRC).read()
    assert src.count(snippet) == 1, f"snippet not unique in oracle.c: {snippet!r}"
    root = os.path.join(base, f"m{idx}")
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(root, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(root, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), root)
    with open(os.path.join(root, "oracle", "oracle.c"), "w") as f:
        f.write(src.replace(snippet, repl))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    build = subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"],
                           cwd=root, env=env, capture_output=True, text=True, timeout=300)
    if build.returncode != 0:
        return "build failed: " + build.stderr[-400:]
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join("tests", pin)], cwd=root, env=env, capture_output=True,
                         text=True, timeout=600)
    return run.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as base:
        with ThreadPoolExecutor(max_workers=4) as pool:
            futs = [pool.submit(_run_mutant, base, i, snip, repl, pin)
                    for i, (_, snip, repl, pin) in enumerate(MUTANTS)]
            results = [f.result() for f in futs]
    bad = [(name, r) for (name, *_), r in zip(MUTANTS, results) if r != 1]
    assert not bad, f"mutants not caught by their pins (pytest status, 1 = failed as required): {bad}"
