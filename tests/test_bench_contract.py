"""The bench's command-line contract: one JSON line with the fields a driver
reads, the roofline and CPU-baseline objects, and a refusal of more than one
GPU. bench.py runs as a child process, as a driver would start it."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_kernel_hash_follows_code_not_comments():
    """The source hash that ties the committed traffic counters to the kernels
    ignores comments, blank lines and trailing spaces, keeps string literals
    (comment markers inside them included), and changes with the code."""
    sys.path.insert(0, ROOT)
    import bench
    a = 'int f() { return 1; } // one\n/* block\n comment */\nconst char *s = "a // b /* c */";\n'
    b = '// other words\nint f() { return 1; }\n\nconst char *s = "a // b /* c */";   \n'
    assert bench.code_text(a) == bench.code_text(b)
    assert '"a // b /* c */"' in bench.code_text(a)
    assert bench.code_text("int x = 1;") != bench.code_text("int x = 2;")
    assert bench.code_text("char c = '/'; // x") == "char c = '/';"
    assert len(bench.kernel_hash("gemm_f32")) == 16


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and not r.stdout.strip()


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.gpu
@pytest.mark.skipif(not _has_gpu(), reason="needs a GPU")
@pytest.mark.parametrize("workload", ["gemm_f32_256", "linear_relu_2047x1376x4096"])
def test_one_json_line_with_every_field(workload):
    r = run_bench("--workload", workload, "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["config"]["workload"] == workload
    rl = d["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 157.3
    assert 0 < rl["frac"] <= 1 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert rl["traffic"] is None or rl["traffic"] > 0
    assert rl["kernel_min_ms"] <= rl["kernel_median_ms"] and rl["kernel_min_ms"] <= rl["kernel_avg_ms"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["unit"] == d["unit"]


@pytest.mark.gpu
@pytest.mark.skipif(not _has_gpu(), reason="needs a GPU")
def test_memory_bound_workload_rates_hbm_bytes():
    """A decode-sized layer (one row of X) is rated against the HBM peak: its
    compulsory bytes per call over the average call time, in GB/s."""
    workload = "linear_relu_nt_1x4096x11008"
    r = run_bench("--workload", workload, "--steps", "5", "--warmup", "2", "--cpu-seconds", "0.2")
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([l for l in r.stdout.splitlines() if l.strip()][0])
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    # X 4096, W 4096 x 11008 and the bias read, Y written, 4 bytes each
    assert rl["bytes_per_launch"] == 4 * (4096 + 4096 * 11008 + 11008 + 11008)
    assert abs(rl["achieved"] - rl["bytes_per_launch"] / (rl["kernel_avg_ms"] * 1e-3) / 1e9) < 1.0
    assert 0 < rl["frac"] <= 1
    assert d["config"]["tile"].endswith("_skinny")


@pytest.mark.gpu
@pytest.mark.skipif(not _has_gpu(), reason="needs a GPU")
def test_default_run_reports_every_configuration():
    """The default run (the 4096^3 headline) also reports the 256^3, 1024^3
    alpha/beta, fused-layer and FP16 8192^3 configurations, each with its time
    per step, TFLOP/s, fraction of its dtype's peak and an oracle sample."""
    r = run_bench("--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5",
                  "--config-cpu-seconds", "0.3", timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["config"]["workload"] == "gemm_f32_4096" and d["roofline"]["peak"] == 157.3
    cf = d["configs"]
    assert set(cf) == {"gemm_f32_256", "gemm_f32_1024_ab", "linear_relu_2047x4096x11008",
                       "gemm_f16f32_8192", "linear_relu_2047x4096x11008_workspace"}
    for name, c in cf.items():
        assert c["ms_per_step"] > 0 and c["tflops"] > 0, name
        assert 0 < c["frac_of_peak"] <= 1 and 0 < c["kernel_frac_of_peak"] <= 1, name
        assert abs(c["tflops"] / c["peak_tflops"] - c["frac_of_peak"]) < 1e-3, name
        if not name.endswith("_workspace"):
            assert c["cpu_baseline"]["kind"] == "oracle" and c["cpu_baseline"]["cores"] >= 1, name
    assert cf["linear_relu_2047x4096x11008_workspace"]["workspace_bytes"] > 0
    assert cf["gemm_f16f32_8192"]["peak_tflops"] == 2516.6
