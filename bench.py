"""Benchmark of one streaming unit of the cached block-causal denoising step.

One step = one 160 ms streaming unit on this GPU's share of the work:
  1. ws_kv_append of the thinker's K/V slice (token-major, all heads of the
     slice, keeping this GPU's head block),
  2. for each denoise step: ws_attn_partial + ws_attn_merge (block-causal
     attention of the unit's latent queries over the cache plus the unit's own
     tokens) and ws_fm_euler_step (x += dt * v),
  3. ws_kv_append of the unit's generated latent K/V (head-major commit).
The cache length is rewound to the same history before every step, so every
step is the same workload. All inputs are resident in HBM before timing.

Prints one JSON line. `value` is attention TFLOP/s over the whole unit (all
denoise steps' algorithmic attention FLOPs / wall time of the unit);
`roofline` is the split-KV attention kernel against the bf16 MFMA peak (or,
for a workload below the ridge point, against HBM bandwidth), its duration
measured with HIP events around each launch on the launch stream.

`--workload v02_history_prefill` measures the multi-unit form instead: one
step is one block-causal call over all 64 cached units (partial + merge).
`--workload joint_rank_share` runs the unit with the audio and video queries
in one call per denoise step, and also times the same unit with one call per
modality (`separate`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
UNIT_BUDGET_MS = 160.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the attention kernel's sources: counter-derived traffic is reported only
# while these are unchanged since the counters were taken
ATTN_SOURCES = [os.path.join(ROOT, "cached_block_causal_amd", "csrc", f)
                for f in ("attn_fwd.hip", "ws_device.hpp", "ws_launch.hpp")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="v02_rank_share")
    p.add_argument("--splits", type=int, default=0, help="0 = library default")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--op-bench", action="store_true",
                   help="instead of the unit step: bandwidth of the cache append (952-token "
                        "40-head slices) and of the Euler update, one JSON line each")
    p.add_argument("--pipeline", action="store_true",
                   help="instead of the fixed unit step: --steps consecutive units on a growing "
                        "cache, each unit's slice appended on a second stream while the previous "
                        "unit denoises; also timed on one stream")
    p.add_argument("--no-side", action="store_true",
                   help="only the named workload's line: no side records of the other "
                        "workloads and ops")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a plain copy (the append kernel) of known size, for "
                        "calibrating HBM byte counters")
    return p.parse_args()


def sources_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch of the attention kernel from committed counter
    runs, only if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sources_sha256_16") != sources_hash(ATTN_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def blas_info():
    """(threads, "vendor version") of the BLAS NumPy uses, for the CPU baseline."""
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover - informational only
        libs = []
    if not libs:
        return os.cpu_count() or 1, "unknown"
    lib = max(libs, key=lambda i: i.get("num_threads", 1))
    return (int(lib.get("num_threads", 1)),
            f"{lib.get('internal_api', '?')} {lib.get('version', '')}".strip())


# parity bar of attention outputs against the oracle (bf16 in, fp32 accumulate)
PARITY_MAX_ABS = 2e-2
PARITY_REL_FRO = 5e-3


class _Parity:
    """Worst error of GPU outputs against the oracle over the problems seen."""

    def __init__(self):
        self.n, self.max_abs, self.rel = 0, 0.0, 0.0

    def add(self, got_f64, want):
        import numpy as np
        diff = got_f64 - want
        self.n += 1
        self.max_abs = max(self.max_abs, float(np.max(np.abs(diff))))
        self.rel = max(self.rel, float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-300)))

    def report(self):
        return {"problems": self.n, "max_abs": self.max_abs, "rel_fro": self.rel,
                "bar": {"max_abs": PARITY_MAX_ABS, "rel_fro": PARITY_REL_FRO},
                "within": self.max_abs <= PARITY_MAX_ABS and self.rel <= PARITY_REL_FRO}


def cpu_baseline(w, budget_s: float, gpu_out=None, ops: bool = True):
    """Time the fp64 oracle on a bounded sample of the same workload: whole
    (denoise step, head) attention problems (all query rows over all keys),
    in step-then-head order, until about budget_s seconds of CPU time.
    gpu_out[step] (host bf16 bits [heads][n_q][D] of the timed run), when
    given, is compared with each problem's oracle result outside the timing."""
    import numpy as np

    import oracle as O
    from workloads import gen as G
    threads, blas = blas_info()
    ids = G.history_unit_ids(w)
    done, flops, elapsed = 0, 0, 0.0
    parity = _Parity()
    hist = {}
    for step in range(w.steps):
        for h in range(w.heads):
            head = [w.head_begin + h]
            if h not in hist:
                hist[h] = G.history_bits(w, head)
            hk, hv = hist[h]
            q, ks, vs, _ = G.step_tensors(w, step, heads=head)
            t0 = time.perf_counter()
            k, v, ku = O.streaming_keys(hk, hv, w.cache_len, ids, ks, vs, w.current_unit)
            qu = np.full(w.n_q, w.current_unit)
            if w.joint:   # audio rows and keys first; video queries also see the audio tokens
                ku[w.cache_len + w.audio_tokens:] += 1
                qu[w.audio_tokens:] += 1
            o = O.attention(q, k, v, qu, ku, 1 / np.sqrt(w.head_dim))
            elapsed += time.perf_counter() - t0
            done += 1
            flops += 4 * w.head_dim * w.visible_pairs()
            if gpu_out is not None:
                parity.add(O.bf16_to_f64(gpu_out[step][h]), o[0])
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
        hist = hist if len(hist) * w.cache_len * w.head_dim * 4 < (2 << 30) else {}
    if not ops:
        return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s",
                "cores": int(threads), "kind": "oracle",
                "sample": f"fp64 NumPy oracle on {done} of {w.steps * w.heads} (denoise step, "
                          f"head) attention problems ({w.n_q} queries x {w.n_keys} keys each), "
                          f"{elapsed:.2f} s of compute",
                "attention_ms_per_problem": round(elapsed / done * 1e3, 2), "blas": blas,
                **({"parity": parity.report()} if gpu_out is not None else {})}
    # the other two steps of the unit, once each: the slice append into a
    # cache of this length and one Euler step of the unit's latent
    ck = np.zeros((w.heads, w.cache_len + w.slice_tokens, w.head_dim), np.uint16)
    sk = np.zeros((w.slice_tokens, w.heads_total, w.head_dim), np.uint16)
    t0 = time.perf_counter()
    O.kv_append(ck, ck, w.cache_len, sk, sk, w.head_begin)
    append_ms = (time.perf_counter() - t0) * 1e3
    n_el = w.n_q * w.heads * w.head_dim
    t0 = time.perf_counter()
    O.fm_euler_state(np.zeros(n_el, np.float32), np.zeros(n_el, np.uint16), w.dt)
    euler_ms = (time.perf_counter() - t0) * 1e3
    return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle on {done} of {w.steps * w.heads} (denoise step, head) "
                      f"attention problems of this workload ({w.n_q} queries x {w.n_keys} keys "
                      f"each), {elapsed:.2f} s of compute; host has {os.cpu_count()} logical CPUs",
            "attention_ms_per_problem": round(elapsed / done * 1e3, 2),
            "append_ms": round(append_ms, 3), "euler_ms": round(euler_ms, 3), "blas": blas,
            **({"parity": parity.report()} if gpu_out is not None else {})}


def roofline(w, attn_ms: list, step_ms: list | None = None) -> dict:
    """The attention kernel against the roofline that bounds it: the bf16
    MFMA peak above the ridge point (peak FLOP/s / peak B/s), HBM below it.
    Both fractions are given, from the average of the timed launches; their
    minimum and 10th/50th/90th percentiles (nearest rank) are reported too.
    `frac`/`achieved` are the split-KV kernel's own launches (the dominant
    kernel); step_ms (the split-KV launch plus its merge, the whole attention
    of a denoise step), when given, is reported beside them as step_*."""
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    srt = sorted(attn_ms)

    def pct(p):
        return srt[max(1, math.ceil(p / 100 * len(srt))) - 1]

    flops, kv = w.attn_flops(), w.attn_kv_bytes()
    tf = flops / (attn_avg_ms * 1e-3) / 1e12
    gbs = kv / (attn_avg_ms * 1e-3) / 1e9
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    hbm = flops / kv < ridge
    # the library runs its narrow kernel for calls with at most 32 queries
    kernel = "attn_narrow_kernel" if w.n_q <= 32 else "attn_partial_kernel"
    r = {"kernel": "%s<%d>" % (kernel, w.head_dim), "bound": "hbm" if hbm else "mfma",
         "achieved": round(gbs if hbm else tf, 2), "peak": PEAK_HBM_GBS if hbm else PEAK_BF16_TFLOPS,
         "unit": "GB/s" if hbm else "TFLOP/s",
         "frac": round((gbs / PEAK_HBM_GBS) if hbm else (tf / PEAK_BF16_TFLOPS), 4),
         "traffic": stored_traffic(w.name),
         "mfma_tflops": round(tf, 2), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
         "kv_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
         "launch_ms_avg": round(attn_avg_ms, 5), "launch_ms_min": round(srt[0], 5),
         "launch_ms_p10": round(pct(10), 5), "launch_ms_p50": round(pct(50), 5),
         "launch_ms_p90": round(pct(90), 5), "launches_timed": len(attn_ms)}
    if step_ms:
        st = sum(step_ms) / len(step_ms)
        r.update({"step_ms_avg": round(st, 5),
                  "step_frac": round((kv / (st * 1e-3) / 1e9 / PEAK_HBM_GBS) if hbm
                                     else (flops / (st * 1e-3) / 1e12 / PEAK_BF16_TFLOPS), 4),
                  "step_what": "split-KV launch + merge launch (events after the merge)"})
    return r


def cpu_baseline_prefill(w, budget_s: float, gpu_out=None):
    """The fp64 oracle on (head, unit) problems of the multi-unit call: the
    queries of one unit over the cache up to that unit's end, the largest
    units first, until about budget_s seconds of CPU time. gpu_out (host
    bf16 bits [heads][n_q][D] of the timed call), when given, is compared
    with each problem's oracle result outside the timing."""
    import numpy as np

    import oracle as O
    from workloads import gen as G
    threads, blas = blas_info()
    ids = G.history_unit_ids(w)
    kend = w.unit_kend()
    done, flops, elapsed = 0, 0, 0.0
    head = [w.head_begin]
    hk, hv = G.history_bits(w, head)
    qb = w.q_unit_begin()
    parity = _Parity()
    for u in reversed(range(w.cached_units)):
        q = G.prefill_queries(w, head, units=[u])
        t0 = time.perf_counter()
        o = O.attention(q, hk[:, :kend[u]], hv[:, :kend[u]], np.full(w.video_tokens, u),
                        ids[:kend[u]], 1 / np.sqrt(w.head_dim))
        elapsed += time.perf_counter() - t0
        done += 1
        if gpu_out is not None:
            parity.add(O.bf16_to_f64(gpu_out[0, qb[u]:qb[u + 1]]), o[0])
        flops += 4 * w.head_dim * w.video_tokens * kend[u]
        if elapsed >= budget_s:
            break
    return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle on {done} of {w.cached_units * w.heads} (head, unit) "
                      f"problems of this call (one unit's {w.video_tokens} queries over the cache "
                      f"up to its end, largest first), {elapsed:.2f} s of compute; host has "
                      f"{os.cpu_count()} logical CPUs",
            "attention_ms_per_problem": round(elapsed / done * 1e3, 2), "blas": blas,
            **({"parity": parity.report()} if gpu_out is not None else {})}


def prefill_bench(w, args) -> None:
    """One step = one multi-unit block-causal call (ws_attn_partial +
    ws_attn_merge) over the whole cached history."""
    import torch

    from cached_block_causal_amd import AttnCall, KVCache, kv_append
    from workloads import gen as G
    from workloads.device import dev_bits, host_bits
    heads = list(range(w.head_begin, w.head_begin + w.heads))
    t_setup = time.perf_counter()
    cache = KVCache(w.heads, w.head_dim, w.capacity)
    for u in range(w.cached_units):                      # history (untimed)
        k, v = G.cache_unit_tokens(w, u, heads)
        kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    q = dev_bits(G.prefill_queries(w))
    call = AttnCall(cache, q, q_unit_begin=w.q_unit_begin(), unit_kend=w.unit_kend(),
                    n_splits=args.splits)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    for _ in range(args.warmup):
        call.partial()
        call.merge()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for a, b in ev:
        a.record()
        call.partial()
        b.record()
        call.merge()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    out = {
        "metric": "attention TFLOP/s of one multi-unit block-causal call (visible query-key "
                  "pairs only), with % of bf16 MFMA peak",
        "value": round(w.attn_flops() / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,1) Q/K/V)",
        "config": {"workload": w.name, "heads": w.heads, "heads_total": w.heads_total,
                   "head_dim": w.head_dim, "n_q": w.n_q, "n_keys": w.n_keys,
                   "units": w.cached_units, "visible_pairs_per_head": w.visible_pairs(),
                   "splits": call.splits},
        "roofline": roofline(w, attn_ms),
        "host_wall_s": round(wall, 3),
        "setup_s": round(setup_s, 2),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_prefill(w, args.cpu_seconds, host_bits(call.out))
    print(json.dumps(out), flush=True)


def pipeline_units(w, units: int):
    """Device inputs of `units` consecutive units after the workload's
    history, and the cache holding that history (room for all units)."""
    import torch

    from cached_block_causal_amd import KVCache, UnitInputs, kv_append
    from workloads import gen as G
    from workloads.device import dev_bits
    heads = list(range(w.head_begin, w.head_begin + w.heads))
    cache = KVCache(w.heads, w.head_dim, w.history_len + units * w.unit_tokens)
    for u in range(w.cached_units):
        k, v = G.cache_unit_tokens(w, u, heads)
        kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    ins = []
    for i in range(units):
        u = w.cached_units + i
        sk, sv = G.cache_unit_tokens(w, u, range(w.heads_total), w.slice_tokens)
        steps = [tuple(dev_bits(t) for t in G.step_tensors(w, s, unit=u)) for s in range(w.steps)]
        x = torch.from_numpy(G.normal_heads(w.seed, G.TAG_X0, u, 0, heads, w.n_q, w.head_dim))
        ins.append(UnitInputs(dev_bits(G.token_major(sk)), dev_bits(G.token_major(sv)), steps,
                              x.to("cuda"), steps[-1][1], steps[-1][2], w.head_begin))
    return cache, ins


def pipeline_bench(w, args) -> None:
    """--steps consecutive units on a growing cache, with the slice appends
    overlapped on a second stream, and the same units on one stream."""
    import torch

    from cached_block_causal_amd import run_units
    cache, ins = pipeline_units(w, args.steps)
    history_len = cache.len
    side = torch.cuda.Stream()
    res = {}
    for overlap in (True, False, True):
        for _ in range(max(1, args.warmup)):
            cache.rewind(history_len)
            run_units(cache, ins, w.dt, overlap, side, args.splits)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cache.rewind(history_len)
        t0.record()
        run_units(cache, ins, w.dt, overlap, side, args.splits)
        t1.record()
        torch.cuda.synchronize()
        res[overlap] = min(res.get(overlap, 1e30), t0.elapsed_time(t1) / args.steps)
    flops = sum(4 * w.head_dim * w.n_q * (w.cache_len + i * w.unit_tokens + w.n_self) * w.heads
                for i in range(args.steps)) * w.steps
    print(json.dumps({
        "metric": "streaming units on a growing cache, slice appends overlapped on a second "
                  "stream: attention TFLOP/s and ms per unit",
        "value": round(flops / (res[True] * args.steps * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res[True], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, as the unit step)",
        "config": {"workload": w.name, "units": args.steps, "first_cache_len": w.cache_len,
                   "last_cache_len": w.cache_len + (args.steps - 1) * w.unit_tokens},
        "one_stream_ms_per_unit": round(res[False], 4),
        "overlap_saving_ms_per_unit": round(res[False] - res[True], 4)}), flush=True)


def calib_copy(steps: int) -> None:
    """Append kernel over a large slice: a plain copy of known size."""
    import torch

    from cached_block_causal_amd import KVCache, kv_append
    heads, d, n = 40, 128, 16384
    cache = KVCache(heads, d, n)
    src_k = torch.zeros((n, heads, d), dtype=torch.bfloat16, device="cuda")
    src_v = torch.zeros_like(src_k)
    for _ in range(steps):
        cache.rewind(0)
        kv_append(cache, src_k, src_v)
    torch.cuda.synchronize()
    nbytes = 2 * n * heads * d * 2
    print(json.dumps({"calib_copy": True, "read_bytes_per_launch": nbytes,
                      "write_bytes_per_launch": nbytes, "launches": steps}))


def _timed(calls: list, reps: int) -> float:
    """GPU seconds per call: the calls are captured once into a HIP graph (the
    library only enqueues kernels; torch's copy_ becomes a copy node) and the
    graph is replayed reps times between two events. Back to back on the GPU
    with no host work in between: a Python call costs more than these short
    kernels take, so timing eager calls would measure the host."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for c in calls:                 # warm-up, outside the capture
            c()
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            for c in calls:
                c()
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * len(calls))


def _bw(op: str, nbytes: int, per_s: float, **extra) -> dict:
    gbs = nbytes / per_s / 1e9
    return {"op": op, **extra, "us_per_call": round(per_s * 1e6, 3), "bytes_per_call": nbytes,
            "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def op_records(steps: int) -> list:
    """HBM bandwidth of the copy-like ops (GPU time per call from HIP-graph
    replays of back-to-back calls), sources and destinations rotating over
    more than the 256 MB last-level cache so that the bytes come from HBM:
      * the unit-end append of the whole performer as one launch
        (ws_kv_append_segments): 920 committed latent tokens, head-major, then
        the next unit's 32-token slice, token-major, all 40 heads (952 rows);
      * the same 952 rows from one token-major slice (ws_kv_append);
      * the plain-copy ceiling for the same bytes measured in the same run:
        one contiguous device-to-device copy of 2 x 952 x 40 x 128 bf16;
      * ws_kv_append of a 16,384-token slice (670 MB moved);
      * ws_fm_euler_step over the whole performer's latent (920 x 40 x 128)."""
    import torch

    from cached_block_causal_amd import (KVCache, fm_euler_step, kv_append,
                                         kv_append_segments)
    heads, d, nbuf = 40, 128, 24
    n_commit, n_slice = 920, 32
    n = n_commit + n_slice
    recs = []
    bf = torch.bfloat16
    commits = [(torch.randn(heads, n_commit, d, device="cuda").to(bf),
                torch.randn(heads, n_commit, d, device="cuda").to(bf)) for _ in range(nbuf)]
    slices = [(torch.randn(n_slice, heads, d, device="cuda").to(bf),
               torch.randn(n_slice, heads, d, device="cuda").to(bf)) for _ in range(nbuf)]
    cache = KVCache(heads, d, n * nbuf)
    nbytes = 2 * (2 * n * heads * d * 2)          # K and V, read + write

    def fused(i):
        def call():
            cache.rewind(i * n)
            (ck, cv), (sk, sv) = commits[i], slices[i]
            kv_append_segments(cache, [(ck, cv, "head", 0), (sk, sv, "token", 0)])
        return call

    per = _timed([fused(i) for i in range(nbuf)], steps)
    recs.append(_bw("ws_kv_append_segments", nbytes, per, tokens=n, heads=heads, head_dim=d,
                    what="unit end: 920 committed tokens (head-major) + 32-token slice "
                         "(token-major) in one launch"))
    tok = [(torch.randn(n, heads, d, device="cuda").to(bf),
            torch.randn(n, heads, d, device="cuda").to(bf)) for _ in range(nbuf)]

    def single(i):
        def call():
            cache.rewind(i * n)
            kv_append(cache, tok[i][0], tok[i][1])
        return call

    per_single = _timed([single(i) for i in range(nbuf)], steps)
    recs.append(_bw("ws_kv_append", nbytes, per_single, tokens=n, heads=heads, head_dim=d,
                    what="one 952-token token-major slice"))
    srcs = [torch.randn(2 * n * heads * d, device="cuda").to(bf) for _ in range(nbuf)]
    dsts = [torch.empty_like(t) for t in srcs]

    def plain(i):
        return lambda: dsts[i].copy_(srcs[i])

    per_copy = _timed([plain(i) for i in range(nbuf)], steps)
    ceil = _bw("plain_copy", nbytes, per_copy, tokens=n, heads=heads, head_dim=d,
               what="contiguous device-to-device copy of the same bytes (torch copy_)")
    recs.append(ceil)
    recs[0]["vs_plain_copy"] = round(per_copy / per, 4)
    recs[1]["vs_plain_copy"] = round(per_copy / per_single, 4)
    del commits, slices, tok, srcs, dsts, cache
    big_n = 16384
    bk = torch.randn(big_n, heads, d, device="cuda").to(bf)
    bv = torch.randn(big_n, heads, d, device="cuda").to(bf)
    big = KVCache(heads, d, big_n)

    def large():
        big.rewind(0)
        kv_append(big, bk, bv)

    recs.append(_bw("ws_kv_append", 2 * (2 * big_n * heads * d * 2), _timed([large], steps),
                    tokens=big_n, heads=heads, head_dim=d))
    del bk, bv, big
    elems = 920 * 40 * 128
    xs = [torch.randn(elems, device="cuda") for _ in range(nbuf)]
    vs = [torch.randn(elems, device="cuda").to(bf) for _ in range(nbuf)]

    def euler(i):
        return lambda: fm_euler_step(xs[i], vs[i], 0.25)

    recs.append(_bw("ws_fm_euler_step", elems * 10, _timed([euler(i) for i in range(nbuf)], steps),
                    elements=elems))
    return recs


def op_bench(steps: int) -> None:
    for r in op_records(steps):
        print(json.dumps(r))


def unit_bench(w, args, cpu_seconds: float, graph: bool = True, cpu_ops: bool = True) -> dict:
    """One streaming unit of workload w, timed over args.steps units (after
    args.warmup): one append launch for the unit's end (the previous unit's
    committed latents, head-major, then this unit's slice, token-major, all
    heads of the slice keeping this GPU's block), then per denoise step
    ws_attn_partial + ws_attn_merge and ws_fm_euler_step. The cache is
    rewound before every unit, so every unit is the same workload."""
    import numpy as np
    import torch

    from cached_block_causal_amd import AttnCall, KVCache, fm_euler_step, kv_append_segments
    from cached_block_causal_amd import kv_append
    from workloads import gen as G
    from workloads.device import dev_bits, host_bits

    heads = list(range(w.head_begin, w.head_begin + w.heads))
    t_setup = time.perf_counter()
    cache = KVCache(w.heads, w.head_dim, w.capacity)
    for u in range(w.cached_units):                      # history (untimed)
        k, v = G.cache_unit_tokens(w, u, heads)
        kv_append(cache, dev_bits(k), dev_bits(v), layout="head")
    # the last history unit's tokens after its slice: re-committed each unit
    ck, cv = G.cache_unit_tokens(w, w.cached_units - 1, heads)
    commit_k = dev_bits(np.ascontiguousarray(ck[:, w.slice_tokens:]))
    commit_v = dev_bits(np.ascontiguousarray(cv[:, w.slice_tokens:]))
    rewind_to = cache.len - commit_k.shape[1]
    sk, sv = G.cache_unit_tokens(w, w.current_unit, range(w.heads_total), w.slice_tokens)
    slice_k, slice_v = dev_bits(G.token_major(sk)), dev_bits(G.token_major(sv))
    segments = [(commit_k, commit_v, "head", 0), (slice_k, slice_v, "token", w.head_begin)]
    cache.rewind(rewind_to)
    kv_append_segments(cache, segments)
    assert cache.len == w.cache_len
    steps_in = [G.step_tensors(w, s) for s in range(w.steps)]
    dq = [dev_bits(t[0]) for t in steps_in]
    dks = [dev_bits(t[1]) for t in steps_in]
    dvs = [dev_bits(t[2]) for t in steps_in]
    dvel = [dev_bits(t[3]) for t in steps_in]
    x = torch.from_numpy(G.x0(w)).to("cuda")
    qb, ke = w.q_unit_begin(), w.unit_kend()
    calls = [AttnCall(cache, dq[0], dks[0], dvs[0], qb, ke, n_splits=args.splits)]
    calls += [AttnCall(cache, dq[s], dks[s], dvs[s], qb, ke, n_splits=args.splits,
                       workspace=calls[0].workspace)      # one workspace for all steps
              for s in range(1, w.steps)]
    splits = calls[0].splits
    sep_calls = None
    if w.joint:
        # the same unit with one call per modality (audio rows first)
        a = w.audio_tokens

        def part(t, lo, hi):
            return t[:, lo:hi].contiguous()

        sep_calls = [[AttnCall(cache, part(dq[s], 0, a), part(dks[s], 0, a), part(dvs[s], 0, a)),
                      AttnCall(cache, part(dq[s], a, w.n_q), part(dks[s], a, w.n_q),
                               part(dvs[s], a, w.n_q))] for s in range(w.steps)]
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    n_attn = args.steps * w.steps
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(n_attn)]

    def unit_step(timed_events=None, per_step=None):
        cache.rewind(rewind_to)
        kv_append_segments(cache, segments)    # previous unit's commit + this unit's slice
        for s in range(w.steps):
            step_calls = [calls[s]] if per_step is None else per_step[s]
            if timed_events is not None:
                timed_events[s][0].record()
            for c in step_calls:
                c.partial()
            if timed_events is not None:
                timed_events[s][1].record()
            for c in step_calls:
                c.merge()
            if timed_events is not None:
                timed_events[s][2].record()
            fm_euler_step(x, dvel[s], w.dt)

    for _ in range(args.warmup):
        unit_step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(args.steps):
        unit_step(ev[i * w.steps:(i + 1) * w.steps])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    attn_ms = [a.elapsed_time(b) for a, b, _ in ev]
    step_ms = [a.elapsed_time(c) for a, _, c in ev]

    flops_step = w.attn_flops()
    value = flops_step * w.steps / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "attention TFLOP/s per 160 ms unit (4 denoise steps), with % of bf16 MFMA "
                  "peak per denoise step and us/unit vs the 160 ms budget",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,1) Q/K/V/velocity, fp32 N(0,1) latent)",
        "config": {"workload": w.name, "heads": w.heads, "heads_total": w.heads_total,
                   "head_dim": w.head_dim, "n_q": w.n_q, "cache_len": w.cache_len,
                   "n_keys": w.n_keys, "denoise_steps": w.steps, "splits": splits,
                   "append_tokens": w.unit_tokens,
                   "append": "one launch: %d committed + %d slice tokens"
                             % (commit_k.shape[1], w.slice_tokens)},
        "roofline": roofline(w, attn_ms, step_ms),
        "us_per_unit": round(ms_per_step * 1e3, 1),
        "unit_budget_frac": round(ms_per_step / UNIT_BUDGET_MS, 5),
        "attention_layers_per_unit_budget": int(UNIT_BUDGET_MS // ms_per_step),
        "host_wall_s": round(wall, 3),
        "setup_s": round(setup_s, 2),
    }
    if sep_calls is not None:
        # the same unit, one call per modality per denoise step
        for _ in range(args.warmup):
            unit_step(per_step=sep_calls)
        torch.cuda.synchronize()
        t0.record()
        for i in range(args.steps):
            unit_step(ev[i * w.steps:(i + 1) * w.steps], per_step=sep_calls)
        t1.record()
        torch.cuda.synchronize()
        sep_ms = t0.elapsed_time(t1) / args.steps
        sep_attn = [a.elapsed_time(b) for a, b, _ in ev]
        out["separate"] = {"ms_per_step": round(sep_ms, 4),
                           "attention_ms_avg": round(sum(sep_attn) / len(sep_attn), 5),
                           "splits": [c.splits for c in sep_calls[0]],
                           "what": "one call for the audio and one for the video queries per "
                                   "denoise step, attention time = both partial launches"}
    if graph:
        out["graph"] = graph_replay(unit_step, args.steps)
    # the same split-KV launches back to back in a graph: no event or host
    # work between launches, so short launches are not inflated by the event
    # pairs (beside, not instead of, the events' figure)
    out["roofline"]["launch_ms_graph"] = round(partial_replay(calls, 10), 5)
    if cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, cpu_seconds, [host_bits(c.out) for c in calls],
                                           ops=cpu_ops)
    return out


# workloads whose records ride along in the default bench line, and the
# oracle time each gets (seconds) for its bounded parity sample
SIDE_WORKLOADS = (("v02_whole_performer", 4.0), ("audio_long_history", 4.0), ("v01_unit", 3.0))


def side_record(rec: dict) -> dict:
    """The parts of a workload's unit record that the default line carries."""
    keep = ("value", "unit", "ms_per_step", "us_per_unit", "unit_budget_frac",
            "attention_layers_per_unit_budget", "setup_s")
    out = {k: rec[k] for k in keep if k in rec}
    out["config"] = {k: rec["config"][k] for k in ("heads", "head_dim", "n_q", "n_keys", "splits")}
    r = rec["roofline"]
    out["roofline"] = {k: r[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac",
                                         "traffic", "mfma_frac", "hbm_frac", "launch_ms_avg",
                                         "launch_ms_p50", "launch_ms_graph", "step_ms_avg",
                                         "step_frac") if k in r}
    if "cpu_baseline" in rec:
        c = rec["cpu_baseline"]
        out["cpu_baseline"] = {k: c[k] for k in ("value", "unit", "cores", "kind", "sample",
                                                 "parity") if k in c}
    return out


def mfma_ceiling(reps: int = 20) -> dict:
    """A dense bf16 product from the vendor library (torch.matmul, 8192^3) on
    the same GPU in the same run: what its matrix cores sustain in practice,
    beside the published peak. Context for the attention kernel's figure, not
    part of the path."""
    import torch
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        c = a @ b
    t1.record()
    torch.cuda.synchronize()
    del a, b, c
    ms = t0.elapsed_time(t1) / reps
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"what": "torch.matmul bf16 8192 x 8192 x 8192 (vendor GEMM library), same run",
            "ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU Ulysses exchange is not built)", file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads as W

    if args.calib_copy:
        calib_copy(args.steps)
        return
    if args.op_bench:
        op_bench(args.steps)
        return
    if args.pipeline:
        pipeline_bench(W.BY_NAME[args.workload], args)
        return

    w = W.BY_NAME[args.workload]
    if w.prefill:
        prefill_bench(w, args)
        return
    out = unit_bench(w, args, 0.0 if args.no_cpu_baseline else args.cpu_seconds)
    if not args.no_side and args.workload == "v02_rank_share" and args.splits == 0:
        # the other targets, in the same run and line: each workload's unit
        # (fewer timed units) with a bounded oracle parity sample, and the ops
        side = argparse.Namespace(**vars(args))
        side.steps, side.warmup = min(args.steps, 10), min(args.warmup, 2)
        out["workloads"] = {}
        for name, secs in SIDE_WORKLOADS:
            rec = unit_bench(W.BY_NAME[name], side, 0.0 if args.no_cpu_baseline else secs,
                             graph=False, cpu_ops=False)
            out["workloads"][name] = side_record(rec)
            torch.cuda.empty_cache()
        out["ops"] = op_records(min(args.steps, 10))
        out["mfma_ceiling"] = mfma_ceiling()
        torch.cuda.empty_cache()
        gemm = out["mfma_ceiling"]["tflops"]
        for r in [out["roofline"]] + [v["roofline"] for v in out["workloads"].values()]:
            if r.get("mfma_tflops") or r.get("bound") == "mfma":
                r["frac_of_gemm"] = round((r.get("mfma_tflops") or r["achieved"]) / gemm, 4)
    print(json.dumps(out), flush=True)


def partial_replay(calls, reps: int) -> float:
    """ms per split-KV launch: one unit's launches (one per denoise step)
    captured back to back into a HIP graph and replayed `reps` times."""
    import torch
    main = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for c in calls:
                c.partial()
    main.wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (reps * len(calls))


def graph_replay(unit_step, steps: int) -> dict:
    """The same unit captured once into a HIP graph (the library only enqueues
    kernels on torch's current stream) and replayed `steps` times: the time per
    unit without per-launch host work. Reported beside, not instead of, the
    eager unit time."""
    import torch
    main = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            unit_step()
    main.wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return {"us_per_unit": round(t0.elapsed_time(t1) / steps * 1e3, 1), "replays": steps,
            "what": "one unit (append, 4 x (partial + merge + Euler), commit) captured once "
                    "and replayed"}


if __name__ == "__main__":
    main()
