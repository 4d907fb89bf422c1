"""One MI355X pipeline stage of patch-level (PipeFusion-style) DiT inference.

The compute path is the HIP library `libpf.so` (built from `csrc/`), reached
through the thin ctypes binding in `binding.py`.  Importing this package does
not load the library; the first binding call does, and raises if it is missing.
"""
from .configs import CONFIGS, StageShape  # noqa: F401
