"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message and exit status 2, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_power_clock_sample_parsing():
    """The amd-smi text bench.py samples: socket power and the highest GFX clock per
    sample; samples without both are skipped."""
    import bench
    block = ("T 1.5\nGPU: 0\n    POWER:\n        SOCKET_POWER: {p} W\n    CLOCK:\n"
             "        GFX_0:\n            CLK: {a} MHz\n            MIN_CLK: 500 MHz\n"
             "        GFX_1:\n            CLK: {b} MHz\n")
    text = block.format(p=1320, a=1850, b=1875) + block.format(p=1335, a=1901, b=1890) + "T 2.0\nerror\n"
    assert bench.parse_smi(text) == [(1320, 1875), (1335, 1901)]
    res = bench.clock_power(bench.parse_smi(text) + [(300, 2400)], 100, 1250.0)
    assert res["samples"] == 2 and res["sclk_mhz_median"] == 1888.0 and res["socket_power_w_median"] == 1327.5
    assert abs(res["roofline_frac_at_measured_clock"] - 1250.0 / (bench.PEAK_BF16_TFLOPS * 1888.0 / 2400.0)) < 1e-4


def test_no_clock_sampler_under_a_profiler(monkeypatch):
    """Under rocprofv3 (ROCPROF* variables in the environment) bench.py starts no
    amd-smi sampler: the profiler's preloaded library would initialise the GPU in
    the sampler's processes, which then replace themselves by exec."""
    import bench
    for name in [n for n in list(bench.os.environ) if n.startswith("ROCPROF")]:
        monkeypatch.delenv(name)
    assert not bench.under_profiler()
    monkeypatch.setenv("ROCPROF_KERNEL_TRACE", "1")
    assert bench.under_profiler()
    res = bench.clock_power([(1320, 1875)], 0, 1250.0, "running under rocprofv3")
    assert res["skipped"] == "running under rocprofv3" and res["samples"] == 0
    assert res["sclk_mhz_median"] is None and res["roofline_frac_at_measured_clock"] is None
