"""Shared-prefix candidate scoring for MI355X (gfx950).

The hot path lives in libjev.so (HIP kernels behind a C ABI, include/jev.h).
`vlm_shared_prefix_amd.jev` is its ctypes binding and
`vlm_shared_prefix_amd.session` a device-memory convenience around it.
Importing the package itself loads nothing, so the build step can run first.
"""
__all__ = ["jev", "session", "build"]
