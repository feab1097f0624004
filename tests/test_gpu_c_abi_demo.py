"""The C ABI from plain C: cached_block_causal_amd/examples/c_abi_demo.c (built
by the package's build step with gcc against libws.so) runs the hand-derived
attention, append and Euler fixtures on the GPU and an error path, and must
print its success line."""
import os
import subprocess

import pytest

from tests.gpu_common import need_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "cached_block_causal_amd", "examples", "c_abi_demo")


@pytest.mark.gpu
def test_c_abi_demo_runs_the_fixtures():
    need_gpu()
    assert os.path.exists(DEMO), "c_abi_demo is not built (run the package build step)"
    print("running c_abi_demo", flush=True)
    r = subprocess.run([DEMO], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_abi_demo ok" in r.stdout
