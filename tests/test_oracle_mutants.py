"""Plant one plausible mistake at a time in a copy of the oracle and check
that the pins catch it (CPU only).

Each mutant is a textual edit of oracle.c -- a transposed index, a dropped
term, a flipped filter, a missing stride, a wrong extent -- compiled with the
oracle's own flags into a temporary library. The pins run in a child process
(a mutant may read outside its arrays) and must report a failure.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from oracle import build as obuild  # noqa: E402

MUTANTS = [
    ("x index: kh and kw swapped",
     "(double)x[xi(n, ci, ho * sh + kh, wo * sw + kw",
     "(double)x[xi(n, ci, ho * sh + kw, wo * sw + kh"),
    ("filter flipped (true convolution instead of correlation)",
     "(double)w[wi(co, ci, kh, kw, Ci, Hf, Wf)]",
     "(double)w[wi(co, ci, Hf - 1 - kh, Wf - 1 - kw, Ci, Hf, Wf)]"),
    ("stride missing on the column axis",
     "(double)x[xi(n, ci, ho * sh + kh, wo * sw + kw",
     "(double)x[xi(n, ci, ho * sh + kh, wo + kw"),
    ("row and column strides swapped",
     "(double)x[xi(n, ci, ho * sh + kh, wo * sw + kw",
     "(double)x[xi(n, ci, ho * sw + kh, wo * sh + kw"),
    ("output width taken with the row stride",
     "int Wo = oracle_out_extent(Wi, Wf, sw);\n    if (Ho == 0 || Wo == 0)\n        return;\n#pragma omp parallel for collapse(2) schedule(dynamic)\n    for (int n = 0; n < N; ++n)\n        for (int co = 0; co < Co; ++co)\n            for (int ho = 0; ho < Ho; ++ho)\n                for (int wo = 0; wo < Wo; ++wo) {\n                    int64_t o",
     "int Wo = oracle_out_extent(Wi, Wf, sh);\n    if (Ho == 0 || Wo == 0)\n        return;\n#pragma omp parallel for collapse(2) schedule(dynamic)\n    for (int n = 0; n < N; ++n)\n        for (int co = 0; co < Co; ++co)\n            for (int ho = 0; ho < Ho; ++ho)\n                for (int wo = 0; wo < Wo; ++wo) {\n                    int64_t o"),
    ("im2win window start uses the row stride",
     "(int64_t)wo * sw * Hf;\n                        for (int kh = 0; kh < Hf; ++kh)\n                            for (int kw = 0; kw < Wf; ++kw)\n                                acc += (double)",
     "(int64_t)wo * sh * Hf;\n                        for (int kh = 0; kh < Hf; ++kh)\n                            for (int kw = 0; kw < Wf; ++kw)\n                                acc += (double)"),
    ("first column of every window dropped",
     "for (int kw = 0; kw < Wf; ++kw) {\n                double p",
     "for (int kw = 1; kw < Wf; ++kw) {\n                double p"),
    ("output extent rounded up",
     "return (in - f) / s + 1;",
     "return (in - f + s - 1) / s + 1;"),
    ("im2win source row uses the column stride",
     "int64_t in = (plane * Hi + (int64_t)ho * sh + kh) * Wi + w;",
     "int64_t in = (plane * Hi + (int64_t)ho * sw + kh) * Wi + w;"),
    ("im2win row stored row by row instead of column by column",
     "int64_t out = ((plane * Ho + ho) * Wi + w) * Hf + kh;",
     "int64_t out = ((plane * Ho + ho) * Hf + kh) * Wi + w;"),
    ("im2win source row ignores the stride",
     "int64_t in = (plane * Hi + (int64_t)ho * sh + kh) * Wi + w;",
     "int64_t in = (plane * Hi + (int64_t)ho + kh) * Wi + w;"),
    ("im2win window read in filter order",
     "acc += (double)win[kw * Hf + kh] *",
     "acc += (double)win[kh * Wf + kw] *"),
    ("absolute-product sum keeps the sign",
     "aacc += fabs(p);",
     "aacc += p;"),
    ("sampled output index decoded with Ho and Wo swapped",
     "int ho = (int)((o / Wo) % Ho);",
     "int ho = (int)((o / Ho) % Wo);"),
    ("output written with rows and columns transposed",
     "int64_t o = (((int64_t)n * Co + co) * Ho + ho) * Wo + wo;",
     "int64_t o = (((int64_t)n * Co + co) * Wo + wo) * Ho + ho;"),
    ("NHWC im2win row stored (kh, w) instead of (w, kh)",
     "int64_t out = ((((int64_t)n * Ho + ho) * Wi + w) * Hf + kh) * Ci + c;",
     "int64_t out = ((((int64_t)n * Ho + ho) * Hf + kh) * Wi + w) * Ci + c;"),
    ("NHWC im2win source row ignores the row stride",
     "int64_t in = (((int64_t)n * Hi + (int64_t)ho * sh + kh) * Wi + w) * Ci + c;",
     "int64_t in = (((int64_t)n * Hi + (int64_t)ho + kh) * Wi + w) * Ci + c;"),
    ("im2col row holds the window in (ci, kw, kh) order",
     "int64_t k = ((int64_t)ci * Hf + kh) * Wf + kw;",
     "int64_t k = ((int64_t)ci * Wf + kw) * Hf + kh;"),
    ("im2col source column ignores the column stride",
     "(int64_t)wo * sw + kw;\n                            memcpy(row",
     "(int64_t)wo + kw;\n                            memcpy(row"),
    ("float-accumulator im2win path multiplies the transposed filter tap",
     "acc += win[kw * Hf + kh] * w[wi(co, ci, kh, kw, Ci, Hf, Wf)];",
     "acc += win[kw * Hf + kh] * w[wi(co, ci, kw, kh, Ci, Hf, Wf)];"),
]


@pytest.mark.parametrize("desc,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(desc, find, repl, tmp_path):
    with open(obuild.SRC) as f:
        src = f.read()
    assert find in src, f"mutation anchor not found: {find!r}"
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(src.replace(find, repl, 1))
    lib = obuild.compile_c(str(mutant_c), str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                       capture_output=True, text=True, timeout=300, env=env, cwd=ROOT)
    assert r.returncode != 0, f"no pin caught: {desc}\n{r.stdout}\n{r.stderr}"
