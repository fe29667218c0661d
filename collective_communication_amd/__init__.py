"""MI355X-native emulated ring AllReduce data path with a lossless bf16 codec.

The compute path is the HIP library ``libhc.so`` (built from ``csrc/`` for
gfx950) behind the C ABI declared in ``include/hc.h``; ``binding`` marshals
torch device tensors to that ABI and nothing more.  Importing this package
does not load the library; the first call does, and it raises when the
library is missing (there is no CPU fallback).
"""

__all__ = ["binding", "inputs"]
