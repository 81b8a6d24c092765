"""The oracle's pins catch plausible mistakes in the oracle itself.

Each case plants one mistake (a dropped term, a wrong sign, a transposed or
shifted index, a wrong exponent bias) into a private copy of the oracle,
rebuilds it and runs the pin suite against the copy: the suite must fail.
A pattern that no longer matches the oracle's source fails too, so that the
list keeps pace with the code it guards. Only the copy is changed; the oracle
under test elsewhere is untouched. Everything runs on the CPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, file under oracle/, text in it, replacement)
MUTANTS = [
    ("last k dropped in the blocked loop", "oracle.c",
     "const int64_t k1 = (K - k0 < KB) ? K : k0 + KB;",
     "const int64_t k1 = (K - k0 < KB) ? K - (K > 3) : k0 + KB;"),
    ("a k chunk summed twice in the blocked loop", "oracle.c",
     "k0 < K; k0 += KB)", "k0 < K; k0 += KB / 2)"),
    ("last k dropped in the per-element loop", "oracle.c",
     "for (int64_t k = 0; k < K; ++k) {\n                const double prod",
     "for (int64_t k = 0; k < K - (K > 3); ++k) {\n                const double prod"),
    ("A read at a shifted k", "oracle.c",
     "la(A, m * lda + k);", "la(A, m * lda + (k + 1) % K);"),
    ("B decoded from the neighbouring column", "oracle.c",
     ": k * ldb + col);", ": k * ldb + (col + 1) % N);"),
    ("B read from the neighbouring column in the blocked loop", "oracle.c",
     "const double p = a * brow[j];", "const double p = a * brow[(j + 1) % nb];"),
    ("A row taken from the neighbouring row in the blocked loop", "oracle.c",
     "const double a = Ad[m * K + k];", "const double a = Ad[((m + 1) % M) * K + k];"),
    ("transposed B decoded with k reversed", "oracle.c",
     "b_trans ? col * ldb + k :", "b_trans ? col * ldb + (K - 1 - k) :"),
    ("per-element loop reads B transposed the wrong way", "oracle.c",
     "b_trans ? n * ldb + k : k * ldb + n", "b_trans ? k * ldb + n : n * ldb + k"),
    ("sample column taken from the wrong position", "oracle.c",
     "m = rows[p], n = cols[p];", "m = rows[p], n = cols[P - 1 - p];"),
    ("beta term subtracted", "oracle.c",
     "r += e->beta * ", "r -= e->beta * "),
    ("alpha dropped", "oracle.c",
     "double r = e->alpha * s;", "double r = s;"),
    ("beta term scaled by alpha too", "oracle.c",
     "r += e->beta * ", "r += e->alpha * e->beta * "),
    ("products summed although alpha is zero", "oracle.c",
     "return !(e->kind == EPI_GEMM && e->alpha == 0.0);", "return 1;"),
    ("bias indexed by row", "oracle.c",
     "e->bias[n];", "e->bias[m % 2];"),
    ("bias added after the ReLU", "oracle.c",
     "    if (e->bias)\n        y += (double)e->bias[n];\n    if (e->act == 1)\n"
     "        y = (y > 0.0) ? y : 0.0;",
     "    if (e->act == 1)\n        y = (y > 0.0) ? y : 0.0;\n"
     "    if (e->bias)\n        y += (double)e->bias[n];"),
    ("ReLU never applied", "oracle.c",
     "if (e->act == 1)", "if (e->act == 2)"),
    ("ReLU gives negative zero", "oracle.c",
     "y = (y > 0.0) ? y : 0.0;", "y = (y > 0.0) ? y : -0.0;"),
    ("magnitude sum without the absolute value", "oracle.c",
     "t[i][j] += fabs(p);", "t[i][j] += p;"),
    ("per-element magnitude sum without the absolute value", "oracle.c",
     "t += fabs(prod);", "t += prod;"),
    ("binary16 exponent bias off by one", "oracle.c",
     "ldexp((double)(f + 1024), e - 25)", "ldexp((double)(f + 1024), e - 24)"),
    ("binary16 implicit bit missing", "oracle.c",
     "ldexp((double)(f + 1024), e - 25)", "ldexp((double)f, e - 25)"),
    ("binary16 subnormal scale wrong", "oracle.c",
     "ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    ("bfloat16 exponent bias off by one", "oracle.c",
     "ldexp((double)(f + 128), e - 134)", "ldexp((double)(f + 128), e - 133)"),
    ("bfloat16 subnormal scale wrong", "oracle.c",
     "ldexp((double)f, -133)", "ldexp((double)f, -134)"),
    ("batch items all use the first B", "__init__.py",
     "gemm(A[i], B[i], alpha", "gemm(A[i], B[0], alpha"),
    ("batch items all use the first C", "__init__.py",
     "None if beta == 0.0 else C[i]", "None if beta == 0.0 else C[0]"),
]


@pytest.mark.parametrize("name,fname,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, fname, old, new):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")

    path = tmp_path / "oracle" / fname
    src = path.read_text(encoding="utf-8")
    assert src.count(old) == 1, f"pattern for '{name}' matches {src.count(old)} times"
    path.write_text(src.replace(old, new), encoding="utf-8")

    env = {k: v for k, v in os.environ.items() if k != "PYTHONPATH"}
    env["OMP_NUM_THREADS"] = "2"
    b = subprocess.run([sys.executable, "-c", "import oracle; oracle.build()"], cwd=tmp_path,
                       env=env, capture_output=True, text=True, timeout=120)
    assert b.returncode == 0, f"mutant '{name}' does not build:\n{b.stderr[-2000:]}"
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle.py", "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=tmp_path, env=env,
                       capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode != 0, f"the pins did not catch: {name}\n{out[-1000:]}"
    assert r.returncode == 1, f"pin suite did not run cleanly for '{name}':\n{out[-2000:]}"
