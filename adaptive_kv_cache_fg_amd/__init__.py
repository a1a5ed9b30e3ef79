"""adaptive_kv_cache_fg_amd -- FastGen's adaptive KV-cache hot path on MI355X.

The compute lives in libfastgen.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/fastgen.h); ``fastgen`` is its Python binding.
"""
from . import fastgen  # noqa: F401
from .fastgen import Cache, FastGenError, Profile, compact, profile, timing_enable, timing_read  # noqa: F401
