"""MI355X (gfx950) 3D-RoPE exact self-attention for the ReGenVC diffusion
transformer decoder.

The computation lives in the HIP library ``libregen_attn.so`` (C ABI in
``include/regen_attn.h``); ``native`` is its ctypes binding, ``sampler`` the
four-step window driver and ``synth`` the seeded synthetic inputs.
"""
from . import synth  # noqa: F401

__all__ = ["native", "sampler", "synth", "build"]
