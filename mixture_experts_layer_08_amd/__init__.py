"""MI355X-native (gfx950) sparse-MoE FFN layer forward.

The layer's steps run in hand-written HIP kernels inside
libmoe_mi355x.so, reached through its C ABI (include/moe.h).  This package is
the thin Python binding: argument marshalling only.  Importing it does not
load the library; the first call does, and raises if the library is missing.
"""
from .synth import CONFIGS, MoEConfig, make_inputs  # noqa: F401

__all__ = ["CONFIGS", "MoEConfig", "make_inputs"]
