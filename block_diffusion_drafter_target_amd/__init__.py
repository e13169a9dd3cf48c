"""MI355X (gfx950) DFlash-style draft step: a C-ABI HIP library and its binding.

    from block_diffusion_drafter_target_amd import Drafter, spec_generate, synth

The compute runs in libdflash.so (HIP kernels); this package marshals torch
device buffers into its entry points (``binding``) and drives the greedy
speculative loop (``drafter``). torch is imported only when a Drafter is used.
"""
from . import binding, synth  # noqa: F401
from .drafter import DeviceTarget, Drafter, spec_generate, spec_generate_device  # noqa: F401

__all__ = ["synth", "binding", "Drafter", "DeviceTarget", "spec_generate", "spec_generate_device"]
