"""The benchmark's command line on the CPU: one GPU only, and a JSON line
that says so otherwise (the GPU legs themselves run on an MI355X)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "3"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_workloads_listed_in_help():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for w in ("qwen3_8b_q32", "square", "pilot_ffn", "expert_ffn", "qwen3_1p7b", "qwen3_8b_down",
              "digraph_qwen3_8b", "pilot_decode_stack", "backward_qwen3_8b", "backward_expert"):
        assert w in r.stdout, w
