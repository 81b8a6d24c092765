"""The CPU-side code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two builds, each in a child process of its own with the sanitizer runtime
preloaded ahead of any library already named in LD_PRELOAD:

* the float64 oracle (oracle.c) built by gcc with -fsanitize=address,undefined,
  running its whole pin suite (tests/test_oracle.py) from a private copy;
* the library's host code (api.hip: argument checks, plan choice, the plan
  queries) built by hipcc with the sanitizers on the host pass only, linked
  with the normally built kernel objects, running the ABI and planner tests
  (tests/test_abi_cpu.py, tests/test_plan_properties.py) through the
  LINEAR_LAYER_LIBRARY override. No GPU is touched: these tests stop at the
  argument checks or the missing device.

Any sanitizer report aborts the child, so the test fails with it.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_layer_amd", "csrc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"sanitizer runtime not found ({' '.join(cmd)})")
    return path


def _env(runtime, **extra):
    env = {k: v for k, v in os.environ.items() if k != "PYTHONPATH"}
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime + (":" + pre if pre else "")
    env.update(SAN_ENV)
    env.update(extra)
    return env


def test_oracle_pins_under_asan_ubsan(tmp_path):
    rt = _runtime(["gcc", "-print-file-name=libasan.so"])
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    flags = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]
    b = subprocess.run([sys.executable, "-c", f"import oracle; oracle.build(extra_flags={flags!r})"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle.py", "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=tmp_path,
                       env=_env(rt, OMP_NUM_THREADS="4"), capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]


def test_host_api_under_asan_ubsan(tmp_path):
    from linear_layer_amd import _build
    rt = _runtime([_build.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"])
    others = [s for s in _build.SOURCES if s != "api.hip"]
    objs = [os.path.join(_build.OBJDIR, os.path.splitext(s)[0] + ".o") for s in others]
    newest = max(os.path.getmtime(os.path.join(CSRC, f)) for f in os.listdir(CSRC))
    if not all(os.path.exists(o) and os.path.getmtime(o) >= newest for o in objs):
        _build.build()
    api_o = str(tmp_path / "api.o")
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", f]
    c = subprocess.run([_build.HIPCC, *_build.CFLAGS, "-g", *san, "-c",
                        os.path.join(CSRC, "api.hip"), "-o", api_o],
                       capture_output=True, text=True, timeout=600)
    assert c.returncode == 0, c.stderr[-2000:]
    lib = str(tmp_path / "liblinear_layer.so")
    ln = subprocess.run([_build.HIPCC, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", api_o,
                         *objs, "-o", lib], capture_output=True, text=True, timeout=600)
    assert ln.returncode == 0, ln.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py",
                        "tests/test_plan_properties.py", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT,
                       env=_env(rt, LINEAR_LAYER_LIBRARY=lib), capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
