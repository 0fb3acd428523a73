"""MI355X-native TMP-shard hot path of the Oases overlapped schedule.

The compute lives in liboases_shard.so (hand-written gfx950 HIP kernels and a
two-stream executor behind a C ABI, see include/oases_shard.h).  ``shard``
is its ctypes binding; ``device`` allocates torch buffers and binds them.
"""
from . import shard  # noqa: F401

__all__ = ["shard"]
