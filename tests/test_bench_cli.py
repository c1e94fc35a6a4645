"""bench.py's command line on the CPU: more than one GPU is refused with a
message (nothing in this build runs on several GPUs), and the help text
names every workload."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_several_gpus_are_refused():
    r = run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_workloads():
    r = run("--help")
    assert r.returncode == 0
    for name in ("llama2_7b", "llama2_7b_skinny", "llama2_7b_skinny_program", "llama2_13b_g128", "llama2_13b_g128_program",
                 "llama3_8b_prefill", "--layout", "--no-extra", "--counter-pass"):
        assert name in r.stdout
