"""Stream Batch denoising on MI355X (gfx950): HIP kernels behind a C ABI.

``libsdstream.so`` (built by ``streaming_diffusion_amd.build``) holds every
step of the path; ``_lib`` binds its C ABI with ctypes and ``runner`` places
weights and workspace in device memory with torch.
"""
from . import _lib  # noqa: F401

__all__ = ["_lib"]
