"""The benchmark's command line on the CPU: a request for more than one GPU ends with a
message and status 2 before anything touches a GPU."""
import pathlib
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""
