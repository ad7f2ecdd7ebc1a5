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
