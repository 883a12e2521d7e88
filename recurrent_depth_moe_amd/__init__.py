"""Looped Recurrent-Block forward on MI355X (gfx950): HIP kernels behind the
C ABI of include/rdt.h, with a thin ctypes binding."""

from .binding import (Block, RdtError, kv_cache_bytes, lib, make_config, weights_to_device,  # noqa: F401
                      workspace_bytes, workspace_offset)
