"""bench.py's command line on the CPU: it measures one GPU only, and says so."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_modes():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--pipeline", "--op-bench",
                 "--calib-copy", "--no-cpu-baseline", "--no-side"):
        assert flag in r.stdout


def test_roofline_block_fields_and_percentiles():
    """The roofline object of a bench line: the bound follows the ridge point
    (MFMA above, HBM below), the fractions divide by the published peaks, and
    the launch percentiles are nearest-rank."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    times = [0.30, 0.31, 0.29, 0.35, 0.32, 0.305, 0.33, 0.28, 0.31, 0.30]
    r = bench.roofline(W.BY_NAME["v02_rank_share"], times)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == bench.PEAK_BF16_TFLOPS
    avg = sum(times) / len(times)
    assert abs(r["achieved"] - 291.5e9 * 1.0 / (avg * 1e-3) / 1e12) / r["achieved"] < 1e-3
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-4
    assert (r["launch_ms_min"], r["launch_ms_p10"], r["launch_ms_p50"], r["launch_ms_p90"]) == \
        (0.28, 0.28, 0.305, 0.33)
    assert r["launches_timed"] == 10
    s = bench.roofline(W.BY_NAME["v02_rank_share"], times, [t + 0.01 for t in times])
    assert abs(s["step_ms_avg"] - (avg + 0.01)) < 1e-9 and s["step_frac"] < s["frac"]
    a = bench.roofline(W.BY_NAME["audio_long_history"], [0.8])
    assert a["bound"] == "hbm" and a["unit"] == "GB/s" and a["kernel"].startswith("attn_narrow")
    assert abs(a["achieved"] - W.BY_NAME["audio_long_history"].attn_kv_bytes() / 0.8e-3 / 1e9) < 0.1
