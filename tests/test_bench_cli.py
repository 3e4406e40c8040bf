"""bench.py's command-line contract that can be checked without a GPU: it
measures one GPU only and refuses more, before touching the device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, timeout=120, env=env,
                          cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    res = _run(["--gpus", "2"])
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_a_multi_rank_launch_is_refused():
    res = _run([], {"WORLD_SIZE": "8"})
    assert res.returncode == 2
    assert "WORLD_SIZE=8" in res.stderr


def test_entry_module_has_build_and_smoke():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "graft_entry", os.path.join(ROOT, "__graft_entry__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert callable(mod.build) and callable(mod.smoke)
