"""Consecutive streaming units on one GPU's growing cache, with each unit's
thinker-slice append overlapped with the previous unit's denoising.

The pages' schedule overlaps adjacent units, and each unit's committed
latents condition the later ones ("Wan-Streamer v0.2：更高分辨率，相同延迟",
方法步骤详情; "Technical Summary: Wan-Streamer v0.2", Methodology, "The
Performer"). Unit k on this GPU:
  1. its slice is appended to the cache (this GPU's head block);
  2. each denoise step runs attention over the cache plus the unit's own
     tokens (partial + merge) and the Euler update of the unit's latent;
  3. the unit's latent K/V are committed to the cache.
With `overlap`, every slice append runs on a second stream. Unit k+1's slice
is enqueued right after unit k's commit is enqueued, so the host assigns it
the rows behind the commit, and it runs while unit k still denoises: unit
k's attention reads only rows below its own end and the commit writes the
rows before the slice, so the two streams never touch the same rows. Unit
k+1's first attention waits for its slice with an event.

Host orchestration only (streams, events, argument order); every step runs
in the library's kernels through the binding.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import ops


@dataclass
class UnitInputs:
    """One streaming unit's device tensors (bf16 bits unless noted)."""
    slice_k: torch.Tensor            # token-major [n][H][D] thinker slice
    slice_v: torch.Tensor
    steps: list                      # per denoise step: (q, k_self, v_self, velocity)
    x: torch.Tensor                  # float32 latent share, updated in place
    commit_k: torch.Tensor           # head-major [Hr][n][D] latents committed at the end
    commit_v: torch.Tensor
    head_begin: int = 0              # this GPU's first head in the slice
    outs: list = field(default_factory=list)   # optional per-step attention outputs


def run_units(cache: ops.KVCache, units: list, dt: float, overlap: bool = True,
              side_stream: torch.cuda.Stream | None = None, n_splits: int = 0,
              attn_events: list | None = None) -> None:
    """Enqueue `units` back to back on the current stream (and `side_stream`
    for the slice appends when `overlap`). Nothing is synchronised; the
    cache length advances on the host as the calls are enqueued.
    attn_events[i][s] (optional) is a pair of timing events recorded around
    unit i's step-s attention launch."""
    main = torch.cuda.current_stream()
    side = None
    if overlap:
        side = side_stream if side_stream is not None else torch.cuda.Stream()
        side.wait_stream(main)     # earlier work on the cache comes first

    def append_slice(u: UnitInputs):
        if side is None:
            ops.kv_append(cache, u.slice_k, u.slice_v, head_begin=u.head_begin)
            return None
        with torch.cuda.stream(side):
            ops.kv_append(cache, u.slice_k, u.slice_v, head_begin=u.head_begin)
        ev = torch.cuda.Event()
        ev.record(side)
        return ev

    ready = append_slice(units[0]) if units else None
    for i, u in enumerate(units):
        if ready is not None:
            main.wait_event(ready)
        ws = None
        for s, (q, ks, vs, vel) in enumerate(u.steps):
            out = u.outs[s] if u.outs else None
            call = ops.AttnCall(cache, q, ks, vs, n_splits=n_splits, out=out, workspace=ws)
            ws = call.workspace
            if attn_events is not None:
                attn_events[i][s][0].record()
            call.partial()
            if attn_events is not None:
                attn_events[i][s][1].record()
            call.merge()
            ops.fm_euler_step(u.x, vel, dt)
        ops.kv_append(cache, u.commit_k, u.commit_v, layout="head")
        if i + 1 < len(units):
            ready = append_slice(units[i + 1])
