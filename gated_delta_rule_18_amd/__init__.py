"""MI355X (gfx950) implementation of the Kimi Delta Attention layer recurrence.

The compute path is the C-ABI library ``libkda.so`` (hand-written HIP kernels,
built from ``csrc/``); ``chunk_fwd`` and ``decode_step`` below marshal torch
tensors to it.  Importing this package does not load the library: the first
call does, and it raises if the library is missing.
"""
__version__ = "0.1.0"


def __getattr__(name):
    if name in ("chunk_fwd", "decode_step", "lib", "version", "KdaError", "library_path"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
