"""Tree-summarised (ZHA) decode attention on MI355X (gfx950).

The compute path is libzha.so (HIP kernels behind a C ABI, include/zha.h);
``hierarchical_kv_cache_amd.zha`` is its ctypes binding.
"""
from . import zha  # noqa: F401
from .zha import (Config, Decoder, LeafList, Tree, ZhaError, append, attend, build,  # noqa: F401
                  build_level, dense_attend, new_workspace, route, route_level,
                  workspace_bytes, ws_status)
