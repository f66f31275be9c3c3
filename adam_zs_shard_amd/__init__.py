"""libzshard: the per-shard ZeRO optimizer step on MI355X (gfx950).

The product is the C-ABI shared library built from csrc/ (declared in
include/zshard.h); `zshard` is its ctypes binding.
"""

from . import zshard  # noqa: F401
