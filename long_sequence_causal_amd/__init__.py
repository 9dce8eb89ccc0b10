"""Chunkwise causal linear attention with per-head decay on MI355X (gfx950).

The compute lives in the HIP library ``liblinattn.so`` (C ABI declared in
``include/linattn.h``); ``long_sequence_causal_amd.linattn`` is the thin
ctypes binding over it.  Importing this package loads nothing: the library
is opened on first use, and a missing or unloadable library is an error.
"""

__all__ = ["inputs", "linattn"]
