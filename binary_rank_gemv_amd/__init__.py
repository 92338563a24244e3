"""MI355X (gfx950) implementation of the LittleBit factored binary linear layer.

The compute path lives in ``csrc/`` (HIP kernels behind a C ABI, built into
``_lib/liblittlebit.so``); ``littlebit`` is the thin ctypes binding over that
ABI.  ``synth`` draws seeded synthetic inputs.  Importing the package does not
load the shared library; ``binary_rank_gemv_amd.littlebit`` does, and raises
if it has not been built.
"""

__all__ = ["littlebit", "synth"]
