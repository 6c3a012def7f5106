"""liblowbit: group-scaled binary / ternary matrix products on MI355X (gfx950).

The compute path is the HIP library under ``csrc/`` (C ABI in
``include/lowbit.h``); ``lowbit`` is its thin Python binding.
"""
from . import lowbit  # noqa: F401
