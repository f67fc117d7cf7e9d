"""bench.py on the CPU: the one-GPU guard, the help text and the pool-placement helper."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_modes():
    r = _bench("--help")
    assert r.returncode == 0
    for flag in ("--workload", "--context", "--op", "--eager", "--partition", "--copy-calibration"):
        assert flag in r.stdout


def test_help_lists_the_pool_placement_flag():
    r = _bench("--help")
    assert "--v-offset" in r.stdout


def test_shifted_pools_copy_and_place():
    sys.path.insert(0, ROOT)
    import bench
    k = torch.arange(2 * 16 * 2 * 128, dtype=torch.float32).to(torch.bfloat16).view(2, 16, 2, 128)
    v = -k
    for off in (0, 256, 768):
        kk, vv = bench.shifted_pools(k, v, off)
        assert torch.equal(kk, k) and torch.equal(vv, v)
        assert vv.data_ptr() - kk.data_ptr() == k.numel() * 2 + off
        assert kk.data_ptr() % 16 == 0 and vv.data_ptr() % 16 == 0
    with pytest.raises(ValueError):
        bench.shifted_pools(k, v, 8)
