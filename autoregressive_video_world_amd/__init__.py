"""Streaming block-causal chunk attention over a bounded KV ring, MI355X-native.

The compute lives in ``libwm.so`` (C ABI declared in ``include/wm.h``, HIP
kernels for gfx950 under ``csrc/``); ``binding`` marshals PyTorch tensors and
streams into it.
"""

from .binding import EVICT_RESET, EVICT_SLIDE, EXPORTS, KVRing, RolloutGraph, WMError, lib  # noqa: F401
