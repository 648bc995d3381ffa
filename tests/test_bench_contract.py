"""The parts of bench.py's contract that need no GPU: it refuses more than one GPU (by flag
or by a torchrun world) with a message and exit status 2 before touching torch, and every
workload name it accepts is one of the seeded configurations."""
import os
import subprocess
import sys

import bench
from virtual_expert_routed_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_a_multi_rank_launch_is_refused():
    r = _run([], {"WORLD_SIZE": "4", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_default_workload_and_every_config_are_known(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    assert (args.gpus, args.config) == (1, "c1_decode_bs23")  # one GPU, the headline workload
    for name in ("c0_tiny_f32", "c1_decode_bs23", "c2_decode_bs128_zipf",
                 "c3_prefill_4096_v8064", "c4_prefill_16384_r64", "n2_verify_h6144"):
        cfg = configs.BY_NAME[name]
        # the kernel names bench reports exist for each stage of each configuration
        for st in cfg.stages:
            assert bench.kernel_name(cfg, st, "shrink").startswith(("shrink_kernel<", "shrink_mfma_kernel<"))
            assert bench.kernel_name(cfg, st, "expand").startswith(("expand_kernel<", "expand_mfma_run_kernel<"))
