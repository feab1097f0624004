"""Cached block-causal denoising step for MI355X (gfx950).

The computation lives in libws.so (hand-written HIP kernels behind the C ABI
of include/ws.h). This package holds the kernel sources (csrc/), the build
script and a thin PyTorch binding; importing the binding needs the built
library and raises if it is missing.
"""
__all__ = ["KVCache", "kv_append", "kv_append_segments", "block_causal_attn", "block_causal_attn_noalloc", "AttnCall",
           "attn_default_splits",
           "attn_workspace_bytes", "fm_euler_step", "UnitInputs", "run_units"]


def __getattr__(name):
    if name in ("UnitInputs", "run_units"):
        from . import pipeline
        return getattr(pipeline, name)
    if name in __all__:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
