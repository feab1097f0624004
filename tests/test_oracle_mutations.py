"""Planted mistakes in a copy of the oracle must fail a pin.

Each case copies oracle/ into a temporary directory with one plausible
mistake written into it (a '<' for '<=' in the mask, a dropped scale, a flipped
sign, V and K swapped, a wrong head offset, single-precision or sign-flipped
Euler arithmetic, a wrong bf16 shift, masked keys weighted as if their score
were 0), copies the pin tests beside it, and runs them in a child
process: they must fail. The unmodified copy must pass, so a failure is the
mistake's doing. The repository's own oracle is never touched.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.py")

MUTATIONS = {
    "mask_strict": ("k_unit[None, :] <= q_unit[:, None]", "k_unit[None, :] < q_unit[:, None]"),
    "scale_dropped": ("s = float(scale) * (q @ k.T)", "s = (q @ k.T)"),
    "exp_sign": ("np.exp(s - m)", "np.exp(m - s)"),
    "v_is_k": ("out[hh, r0:r1] = p @ v[hh]", "out[hh, r0:r1] = p @ k[hh]"),
    "head_offset": ("k_src[:, head_begin:head_begin + hr, :]", "k_src[:, 0:hr, :]"),
    "euler_single": ("return x64 + np.float64(np.float32(dt)) * v64",
                     "return (x64.astype(np.float32) + np.float32(dt) * v64.astype(np.float32))"
                     ".astype(np.float64)"),
    "euler_sign": ("return x64 + np.float64(np.float32(dt)) * v64",
                   "return x64 - np.float64(np.float32(dt)) * v64"),
    "bf16_shift": ("<< np.uint32(16)).view", "<< np.uint32(15)).view"),
    "mask_leaks": ("e = np.where(mask, np.exp(s - m), 0.0)",
                   "e = np.exp(np.where(mask, s, 0.0) - m)"),
}

PIN_FILES = ("__init__.py", "conftest.py", "brute.py", "test_oracle_pins.py", "test_golden.py")


def _run_pins(tmp_path, oracle_text):
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), pkg / "__init__.py")
    (pkg / "oracle.py").write_text(oracle_text)
    tests = tmp_path / "tests"
    tests.mkdir()
    for f in PIN_FILES:
        shutil.copy(os.path.join(ROOT, "tests", f), tests / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tests / "golden")
    # the copied conftest puts tmp_path first on sys.path, so `import oracle`
    # finds the copy; everything else (workloads) comes from the repository
    env = dict(os.environ, PYTHONPATH=ROOT)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "-m", "not gpu", "tests"], cwd=tmp_path, env=env,
                          capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes_the_pins(tmp_path):
    with open(ORACLE_SRC) as f:
        r = _run_pins(tmp_path, f.read())
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    with open(ORACLE_SRC) as f:
        src = f.read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation site of {name} not found once"
    r = _run_pins(tmp_path, src.replace(old, new))
    assert r.returncode == 1, f"{name} not caught:\n" + r.stdout[-2000:] + r.stderr[-2000:]
