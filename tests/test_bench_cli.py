"""The benchmark's command line on the host: it refuses more than one GPU before touching any."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_a_multi_rank_launch_is_refused():
    r = _run(env_extra={"WORLD_SIZE": "8"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_workloads_are_listed_in_the_help():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("attn4096", "llama7b", "l70b_b1", "l70b_b16", "mlp_b8", "decode4096", "encode4096",
              "ecdecode4096", "ecgemv4096"):
        assert w in r.stdout
