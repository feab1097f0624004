"""The five synthetic workloads of the cached block-causal denoising step.

Shapes follow the pages' workloads: the v0.1 output of 192x336 and the v0.2
output of 640x368 at 25 FPS in 160 ms streaming units ("Wan-Streamer v0.2:
Higher Resolution, Same Latency", English abstract; technical summary,
Results), with one latent token per 16x16 pixel patch (a reading: the pages
give no stride), thinker K/V slices of 16 or 32 tokens per unit, and a
Ulysses rank holding a contiguous block of 10 of 40 heads (technical summary,
Methodology, "The Performer"). The pages print no tensor sizes; every number
here is a stated reading, and nothing here computes any part of the method.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    heads_total: int        # H: heads in a thinker slice (whole performer)
    heads: int              # Hr: heads held by this GPU (contiguous block)
    head_begin: int         # first head of this GPU's block
    head_dim: int           # D
    video_tokens: int       # latent video tokens per unit
    slice_tokens: int       # thinker K/V slice tokens per unit
    audio_tokens: int       # latent audio tokens per unit
    cached_units: int       # complete prior units in the cache
    query: str              # "video" or "audio": which latent is denoised;
                            # "joint": the unit's audio, then video, queries in
                            # one call; "prefill": every cached unit's video
                            # tokens at once
    history_audio: bool     # history units also hold their audio tokens
    data_scale: float = 1.0  # Q/K/V ~ N(0,1) * data_scale before bf16 rounding
    steps: int = 4          # denoise steps per unit
    dt: float = 0.25        # Euler step size
    seed: int = 0
    unit_ms: float = 160.0  # streaming unit length

    # ---- derived sizes (pure bookkeeping) ----
    @property
    def unit_tokens(self) -> int:
        """Tokens one complete prior unit occupies in the cache: its slice,
        then its committed video latent (and audio latent where kept)."""
        return (self.slice_tokens + self.video_tokens
                + (self.audio_tokens if self.history_audio else 0))

    @property
    def prefill(self) -> bool:
        """Multi-unit form: the queries of all cached units in one call, each
        unit seeing the cache up to its own end (no current unit)."""
        return self.query == "prefill"

    @property
    def history_len(self) -> int:
        return self.cached_units * self.unit_tokens

    @property
    def cache_len(self) -> int:
        """Valid cache rows at attention time: history + current slice."""
        return self.history_len + (0 if self.prefill else self.slice_tokens)

    @property
    def joint(self) -> bool:
        """Audio and video queries of the current unit in one call: rows
        [0, audio) are audio, the rest video; the own tokens are ordered the
        same way."""
        return self.query == "joint"

    @property
    def n_q(self) -> int:
        if self.prefill:
            return self.cached_units * self.video_tokens
        if self.joint:
            return self.audio_tokens + self.video_tokens
        return self.video_tokens if self.query == "video" else self.audio_tokens

    @property
    def n_self(self) -> int:
        """The current unit's own latent tokens of the denoised modality."""
        return 0 if self.prefill else self.n_q

    def q_unit_begin(self) -> list:
        """First query row of every query group, then n_q (the call's unit
        table)."""
        if self.prefill:
            return [u * self.video_tokens for u in range(self.cached_units + 1)]
        if self.joint:
            return [0, self.audio_tokens, self.n_q]
        return [0, self.n_q]

    def unit_kend(self) -> list:
        """Keys visible to each query group: a unit sees the cache up to its
        own end (streaming: everything, its own tokens included). Joint: the
        audio queries see the cache and the unit's audio tokens, the video
        queries also the unit's video tokens."""
        if self.prefill:
            return [(u + 1) * self.unit_tokens for u in range(self.cached_units)]
        if self.joint:
            return [self.cache_len + self.audio_tokens, self.n_keys]
        return [self.n_keys]

    @property
    def n_keys(self) -> int:
        return self.cache_len + self.n_self

    @property
    def current_unit(self) -> int:
        return self.cached_units

    @property
    def latent_elems(self) -> int:
        """Euler state size for one unit on this GPU: its share [Hr][Nq][D]."""
        return self.heads * self.n_q * self.head_dim

    @property
    def capacity(self) -> int:
        """Cache capacity used by tests and the bench: room for the history,
        the current slice and the current unit's committed latents."""
        return self.history_len + self.unit_tokens

    def visible_pairs(self) -> int:
        """(query, key) pairs one head's call computes (masked pairs excluded)."""
        qb, ke = self.q_unit_begin(), self.unit_kend()
        return sum((qb[u + 1] - qb[u]) * ke[u] for u in range(len(ke)))

    def attn_flops(self) -> int:
        """Algorithmic attention FLOPs of one call: 4*D per visible (query,
        key) pair per head (QK^T and PV)."""
        return 4 * self.head_dim * self.visible_pairs() * self.heads

    def attn_kv_bytes(self) -> int:
        """K and V bytes of one denoise step, each visible key read once."""
        return 2 * self.heads * self.n_keys * self.head_dim * 2


TINY = Workload(
    name="tiny",
    description="4 heads, head_dim 64, 2 cached units + current unit; 252 video "
                "tokens (192x336 at 16x stride) + 16 slice tokens per unit; "
                "Q/K/V ~ N(0,1)/8",
    heads_total=4, heads=4, head_begin=0, head_dim=64,
    video_tokens=252, slice_tokens=16, audio_tokens=0, cached_units=2,
    query="video", history_audio=False, data_scale=1.0 / 8.0)

V01_UNIT = Workload(
    name="v01_unit",
    description="v0.1-resolution unit: 24 heads, head_dim 128, 252 video + 32 "
                "slice tokens per unit, 32 cached units (9,372 keys)",
    heads_total=24, heads=24, head_begin=0, head_dim=128,
    video_tokens=252, slice_tokens=32, audio_tokens=0, cached_units=32,
    query="video", history_audio=False)

V02_RANK = Workload(
    name="v02_rank_share",
    description="v0.2 one-rank share: 640x368 at 16x stride = 920 video tokens "
                "per unit, 10 of 40 heads (4-way head split), head_dim 128, 32 "
                "slice tokens per unit, 64 cached units (61,880 keys)",
    heads_total=40, heads=10, head_begin=0, head_dim=128,
    video_tokens=920, slice_tokens=32, audio_tokens=0, cached_units=64,
    query="video", history_audio=False)

V02_WHOLE = Workload(
    name="v02_whole_performer",
    description="v0.2 whole performer on one GPU: 920 video tokens per unit, all "
                "40 heads, head_dim 128, 32 slice tokens, 64 cached units",
    heads_total=40, heads=40, head_begin=0, head_dim=128,
    video_tokens=920, slice_tokens=32, audio_tokens=0, cached_units=64,
    query="video", history_audio=False)

AUDIO_LONG = Workload(
    name="audio_long_history",
    description="unsharded audio path: 4 audio query tokens per unit, 40 heads, "
                "head_dim 128, 256 cached units of 920 video + 32 slice + 4 audio "
                "tokens (244,772 keys)",
    heads_total=40, heads=40, head_begin=0, head_dim=128,
    video_tokens=920, slice_tokens=32, audio_tokens=4, cached_units=256,
    query="audio", history_audio=True)

V02_PREFILL = Workload(
    name="v02_history_prefill",
    description="multi-unit block-causal attention at scale: re-encode the v0.2 rank "
                "share's 64-unit history in one call, the 920 video tokens of every "
                "unit as queries over the cache up to that unit's end (58,880 queries, "
                "60,928 keys, 10 heads, head_dim 128)",
    heads_total=40, heads=10, head_begin=0, head_dim=128,
    video_tokens=920, slice_tokens=32, audio_tokens=0, cached_units=64,
    query="prefill", history_audio=False, steps=1)

JOINT_RANK = Workload(
    name="joint_rank_share",
    description="the unit's 4 audio and 920 video queries in one call on one rank's 10 of "
                "40 heads over the 256-unit history of 920 video + 32 slice + 4 audio tokens "
                "(245,692 keys): one pass over the cache serves both modalities",
    heads_total=40, heads=10, head_begin=0, head_dim=128,
    video_tokens=920, slice_tokens=32, audio_tokens=4, cached_units=256,
    query="joint", history_audio=True)

ALL = [TINY, V01_UNIT, V02_RANK, V02_WHOLE, AUDIO_LONG, V02_PREFILL, JOINT_RANK]
STREAMING = [w for w in ALL if not w.prefill]   # the per-unit denoising step
BY_NAME = {w.name: w for w in ALL}
