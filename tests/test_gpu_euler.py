"""ws_fm_euler_step on the GPU against the oracle's Euler update."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from workloads import gen as G
from tests.gpu_common import MAX_ABS, REL_FRO, dev_bits, need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w", W.STREAMING, ids=[w.name for w in W.STREAMING])
def test_unit_denoise_states_bit_exact(w):
    """All denoise steps of one unit: every intermediate float32 state equals
    the oracle's correctly rounded x + dt*v (hence also the tolerance bar)."""
    need_gpu()
    from cached_block_causal_amd import fm_euler_step
    print(f"euler {w.name}", flush=True)
    x0 = G.x0(w)
    vel = [G.step_tensors(w, s)[3] for s in range(w.steps)]
    x = torch.from_numpy(x0.copy()).to("cuda")
    want = x0
    for s in range(w.steps):
        fm_euler_step(x, dev_bits(vel[s]), w.dt)
        want64 = O.fm_euler_step(want, vel[s], w.dt)
        want = want64.astype(np.float32)
        got = x.cpu().numpy()
        diff = got.astype(np.float64) - want64
        assert np.max(np.abs(diff)) <= MAX_ABS
        assert np.linalg.norm(diff) <= REL_FRO * np.linalg.norm(want64)
        assert np.array_equal(got, want), f"step {s}"


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1023, 4099])
def test_ragged_lengths_and_dt(n):
    need_gpu()
    from cached_block_causal_amd import fm_euler_step
    rng = np.random.default_rng(n)
    x0 = rng.standard_normal(n).astype(np.float32) * 3
    v = G.bf16_rne_bits(rng.standard_normal(n).astype(np.float32))
    for dt in (0.25, -0.1, 0.0):
        x = torch.from_numpy(x0.copy()).to("cuda")
        fm_euler_step(x, dev_bits(v), dt)
        assert np.array_equal(x.cpu().numpy(), O.fm_euler_state(x0, v, dt)), dt
