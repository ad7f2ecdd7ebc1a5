"""bench.py's command line on the host: it measures one GPU and says so for
any other count, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""


def test_workload_names_are_listed_in_help():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for w in ("650m-decode", "1.5b-prefill", "4b-decode", "4b-prefill", "long-decode-b1", "long-decode-b8",
              "tiny-decode", "hgqa-decode", "kivi-decode", "1.5b-prefill-bwd", "1.5b-ttft"):
        assert w in r.stdout


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_for_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_recorded_traffic_only_for_the_profiled_source(monkeypatch):
    """roofline.traffic comes from the committed counter summary, and only
    while the kernel source it was taken on is unchanged."""
    bench = _bench_module()
    text = open(os.path.join(ROOT, "profiles", "decode_650m_bf16_hbm_traffic.txt"), encoding="utf-8").read()
    fields = dict(l.split(":", 1) for l in text.splitlines() if ":" in l and not l.startswith("#"))
    recorded = fields["source_sha256_16"].strip()
    monkeypatch.setattr(bench, "source_sha", lambda *names: recorded)
    t = bench.recorded_traffic("decode")
    assert t == int(fields["traffic_bytes_per_launch"])
    assert 1.0 <= t / int(fields["algorithmic_bytes_per_launch"]) < 1.1
    monkeypatch.setattr(bench, "source_sha", lambda *names: "0" * 16)
    assert bench.recorded_traffic("decode") is None


def test_median_and_percentiles():
    bench = _bench_module()
    st = bench._stats([float(x) for x in (9, 1, 5, 3, 7, 2, 8, 4, 6, 10)])
    assert st["median_ms"] == 5.5 and st["reps"] == 10
    assert abs(st["p10_ms"] - 1.9) < 1e-12 and abs(st["p90_ms"] - 9.1) < 1e-12
    assert st["mean_ms"] == 5.5 and st["min_ms"] == 1.0 and st["max_ms"] == 10.0


def test_clock_summary_from_sampler_output():
    """The device block's clocks are parsed from rocm-smi's JSON lines; a
    sampler that saw nothing says so instead of failing."""
    import json
    bench = _bench_module()

    class Proc:
        def __init__(self, lines):
            self.lines = lines

        def terminate(self):
            pass

        def kill(self):
            pass

        def communicate(self, timeout=None):
            return "\n".join(self.lines), None

    card = {"card0": {"sclk clock speed:": "(2400Mhz)", "mclk clock speed:": "(1900Mhz)", "sclk clock level:": "1"}}
    low = {"card0": {"sclk clock speed:": "(1500Mhz)", "mclk clock speed:": "(1900Mhz)"}}
    lines = [json.dumps({"t": i, "out": json.dumps(c), "err": ""}) for i, c in enumerate((card, low, card))]
    out = bench.stop_clock_sampler(Proc(lines))
    assert out["clocks"]["sclk_mhz"] == {"min": 1500, "median": 2400, "max": 2400}
    assert out["clocks"]["mclk_mhz"]["median"] == 1900 and out["clock_samples"] == 3
    out = bench.stop_clock_sampler(Proc([json.dumps({"t": 0, "out": "", "err": "no rocm-smi"})]))
    assert out["clocks"].startswith("unavailable")
