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
    while the decode source it was taken on is unchanged."""
    bench = _bench_module()
    text = open(os.path.join(ROOT, "profiles", "decode_650m_bf16_hbm_traffic.txt"), encoding="utf-8").read()
    fields = dict(l.split(":", 1) for l in text.splitlines() if ":" in l and not l.startswith("#"))
    recorded = fields["source_sha256_16"].strip()
    monkeypatch.setattr(bench, "decode_source_sha", lambda: recorded)
    t = bench.recorded_traffic()
    assert t == int(fields["traffic_bytes_per_launch"])
    assert 1.0 <= t / int(fields["algorithmic_bytes_per_launch"]) < 1.1
    monkeypatch.setattr(bench, "decode_source_sha", lambda: "0" * 16)
    assert bench.recorded_traffic() is None
