"""bench.py's command line on the host: asking for more than one GPU, directly
or through a torch.distributed launch, stops with exit status 2 and a message
before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, extra_env=None):
    env = dict(os.environ)
    env.update(extra_env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_distributed_launch_is_refused():
    r = run_bench(["--gpus", "1"], {"WORLD_SIZE": "4", "RANK": "0"})
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    # only rank 0 speaks
    r = run_bench(["--gpus", "1"], {"WORLD_SIZE": "4", "RANK": "3"})
    assert r.returncode == 2
    assert r.stderr == ""
