"""MI355X-native expert-parallel routing layout, dispatch pack and combine.

The hot path runs in hand-written gfx950 HIP kernels behind a C ABI
(``include/ep.h``, ``libep.so``); this package is a thin binding over it.
Importing it requires the built library -- there is no CPU fallback.
"""

from . import abi  # noqa: F401  (raises ImportError when libep.so is missing)
from .buffer import Buffer, Handle, Layout, LowLatencyHandle  # noqa: F401

__all__ = ["Buffer", "Handle", "Layout", "LowLatencyHandle", "abi"]
