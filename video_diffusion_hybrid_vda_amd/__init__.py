"""Video DeltaNet (VDN) hybrid attention forward for MI355X (gfx950).

The compute path lives in the HIP shared library libvdn.so (C ABI declared in
include/vdn.h); `vdn` is its thin ctypes binding.  Nothing is loaded at
import time: `from video_diffusion_hybrid_vda_amd import vdn` loads the
library and fails loudly if it has not been built.
"""
__all__ = ["synth", "vdn"]
