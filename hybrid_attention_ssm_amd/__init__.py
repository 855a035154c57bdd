"""libhymba_hh: the Hymba hybrid-head layer's hot path on MI355X (gfx950).

The compute lives in the HIP library `libhymba_hh.so` (C ABI declared in
include/hh.h); `binding` marshals torch device tensors into those calls.
"""
from . import configs, synth  # noqa: F401

__all__ = ["configs", "synth"]
