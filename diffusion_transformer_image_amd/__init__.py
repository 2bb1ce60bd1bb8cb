"""Z-Image S3-DiT denoiser forward on AMD MI355X (gfx950).

The engine is the C-ABI library ``libzimg_dit.so`` (include/zimg_dit.h,
include/zimg_ops.h) with hand-written HIP kernels; this package is its thin
ctypes binding plus the FlowMatch Euler drivers (plain and with
classifier-free guidance).
"""

from . import binding
from .binding import DiT, ZimgError, config, manifest
from .sampler import cfg_euler_loop, euler_loop, schedule

__all__ = ["binding", "DiT", "ZimgError", "config", "manifest", "euler_loop", "cfg_euler_loop", "schedule"]
