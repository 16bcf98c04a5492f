"""Host-side logic of bench.py (no GPU): the one-GPU contract, the amd-smi
clock parser, and the committed counter summary's entry for the bench
kernel."""
import json
import os
import subprocess
import sys
import types

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _fake_run(stdout):
    return lambda *a, **k: types.SimpleNamespace(stdout=stdout, returncode=0)


def test_smi_clock_parser(monkeypatch):
    clk = lambda v: {"value": v, "unit": "MHz"}
    gfx = {f"gfx_{i}": {"clk": clk(2100 + i), "min_clk": clk(500), "max_clk": clk(2400),
                        "clk_locked": "DISABLED", "deep_sleep": "ENABLED"} for i in range(8)}
    gfx["mem_0"] = {"clk": clk(2000), "min_clk": clk(2000), "max_clk": clk(2000),
                    "clk_locked": "N/A", "deep_sleep": "DISABLED"}
    gfx["fclk_0"] = {"clk": "N/A", "min_clk": "N/A", "max_clk": "N/A"}
    monkeypatch.setattr(subprocess, "run", _fake_run(json.dumps({"gpu_data": [{"gpu": 0, "clock": gfx}]})))
    got = bench.smi_clocks()
    assert got == {"gfx_mhz_median": 2104, "gfx_min_mhz": 500, "gfx_max_mhz": 2400,
                   "gfx_locked": "DISABLED", "mem_mhz": 2000}


def test_smi_clock_parser_failures(monkeypatch):
    monkeypatch.setattr(subprocess, "run", _fake_run("not json"))
    assert bench.smi_clocks() is None

    def missing(*a, **k):
        raise FileNotFoundError("amd-smi")
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench.smi_clocks() is None


def test_power_clock_parser():
    """The socket power and the median of the XCDs' shader clocks, from the
    layout `amd-smi metric --power --clock --json` prints (voltages and
    throttle status reported as N/A; non-gfx clocks ignored)."""
    clk = lambda v: {"value": v, "unit": "MHz"}
    clock = {f"gfx_{i}": {"clk": clk(1880 + i), "min_clk": clk(500), "max_clk": clk(2400)} for i in range(8)}
    clock["mem_0"] = {"clk": clk(2000)}
    clock["fclk_0"] = {"clk": "N/A"}
    power = {"socket_power": {"value": 1244, "unit": "W"}, "gfx_voltage": "N/A", "throttle_status": "N/A"}
    text = json.dumps({"gpu_data": [{"gpu": 1, "power": {"socket_power": {"value": 99, "unit": "W"}}, "clock": clock},
                                     {"gpu": 0, "power": power, "clock": clock}]})
    assert bench.parse_power_clock(text) == (1244, 1883.5)
    assert bench.parse_power_clock(text, index=1) == (99, 1883.5)
    # a list at the top level, as older versions of the tool print
    assert bench.parse_power_clock(json.dumps([{"gpu": 0, "power": power, "clock": clock}])) == (1244, 1883.5)
    # missing readings and unparsable output
    assert bench.parse_power_clock(json.dumps({"gpu_data": [{"gpu": 0, "power": {"socket_power": "N/A"},
                                                             "clock": clock}]})) is None
    assert bench.parse_power_clock(json.dumps({"gpu_data": [{"gpu": 0, "power": power, "clock": {}}]})) is None
    assert bench.parse_power_clock(json.dumps({"gpu_data": [{"gpu": 3, "power": power, "clock": clock}]})) is None
    assert bench.parse_power_clock("not json") is None


def test_committed_counters_cover_the_bench_kernel():
    """The committed counter summary has the bench kernel's entry, at least
    its algorithmic bytes.  When it was taken from other kernel sources than
    the tree's, bench.py reports the traffic as null, and this check is
    skipped until the counters are taken again."""
    import pytest

    import dense_gemm_amd as dg
    k = dg.dg_select_kernel(0, 0, 4096, 4096, 4096, 256, 4096, 256, 4096, 256, 4096, dg.DG_F32)
    traffic = bench.measured_traffic(k, 0, 0, 4096, 4096)
    if traffic is None:
        pytest.skip("profiles/hbm_traffic.txt was taken from other kernel sources")
    # at least the algorithmic bytes (A and B read once, C written once)
    assert traffic >= 3 * 4096 * 4096 * 4


def test_amd_smi_children_skipped_under_profiler(monkeypatch):
    """rocprofv3 exports ROCPROF_* variables; with one set, the clock reading
    starts no amd-smi child process and returns None."""
    for k in [k for k in os.environ if k.startswith("ROCPROF_")]:
        monkeypatch.delenv(k)
    assert not bench.under_profiler()
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp/x")
    assert bench.under_profiler()

    def no_child(*a, **k):
        raise AssertionError("amd-smi started under a profiler")
    monkeypatch.setattr(subprocess, "run", no_child)
    assert bench.smi_clocks() is None
