"""Consecutive streaming units on one GPU's growing cache, each unit's end
(its committed latents and the next unit's thinker slice) written with one
append launch that runs beside the unit's last denoise step.

The pages' schedule overlaps adjacent units, and each unit's committed
latents condition the later ones ("Wan-Streamer v0.2：更高分辨率，相同延迟",
方法步骤详情; "Technical Summary: Wan-Streamer v0.2", Methodology, "The
Performer"). Unit k on this GPU:
  1. each denoise step runs attention over the cache plus the unit's own
     tokens (partial + merge) and the Euler update of the unit's latent;
  2. at its end, the unit's latent K/V (the last step's own tokens) and unit
     k+1's slice are appended, in that order, with one launch
     (ws_kv_append_segments). Unit 0's slice is appended first on its own.
With `overlap`, the appends run on a second stream: the unit-end append is
enqueued right after the last step's attention pass, so it runs beside that
pass, its merge and the Euler update. The host enqueues that pass first, so
the pass covers exactly the rows up to the unit's slice, and the append
writes the rows behind them, which no pass of unit k reads. Unit k+1's first
attention waits for the append with an event. Without `overlap`, everything
runs in that order on one stream.

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
    for the appends when `overlap`). Nothing is synchronised; the cache
    length advances on the host as the calls are enqueued.
    attn_events[i][s] (optional) is a pair of timing events recorded around
    unit i's step-s attention launch."""
    main = torch.cuda.current_stream()
    side = None
    if overlap:
        side = side_stream if side_stream is not None else torch.cuda.Stream()
        side.wait_stream(main)     # earlier work on the cache comes first

    def append(segments):
        if side is None:
            ops.kv_append_segments(cache, segments)
            return None
        with torch.cuda.stream(side):
            ops.kv_append_segments(cache, segments)
        ev = torch.cuda.Event()
        ev.record(side)
        return ev

    ready = None
    if units:
        u0 = units[0]
        ready = append([(u0.slice_k, u0.slice_v, "token", u0.head_begin)])
    for i, u in enumerate(units):
        if ready is not None:
            main.wait_event(ready)
        ws = None
        # unit end: this unit's latents, then the next unit's slice
        end = [(u.commit_k, u.commit_v, "head", 0)]
        if i + 1 < len(units):
            n = units[i + 1]
            end.append((n.slice_k, n.slice_v, "token", n.head_begin))
        last = len(u.steps) - 1
        for s, (q, ks, vs, vel) in enumerate(u.steps):
            out = u.outs[s] if u.outs else None
            call = ops.AttnCall(cache, q, ks, vs, n_splits=n_splits, out=out, workspace=ws)
            ws = call.workspace
            if attn_events is not None:
                attn_events[i][s][0].record()
            call.partial()
            if attn_events is not None:
                attn_events[i][s][1].record()
            if s == last and side is not None:
                ready = append(end)          # beside this pass, merge and Euler
            call.merge()
            ops.fm_euler_step(u.x, vel, dt)
        if side is None:
            append(end)
