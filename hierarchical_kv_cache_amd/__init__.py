"""Tree-summarised (ZHA) decode attention on MI355X (gfx950).

The compute path is libzha.so (HIP kernels behind a C ABI, include/zha.h);
``hierarchical_kv_cache_amd.zha`` is its ctypes binding.  Names are resolved on
first use so that ``python -m hierarchical_kv_cache_amd.buildlib`` can rebuild the
library; using any of them without a built library raises ImportError.
"""
_API = ("Config", "Decoder", "LeafList", "Tree", "ZhaError", "append", "attend", "attend_static", "build",
        "build_level", "dense_attend", "new_workspace", "p_schedule", "route", "route_level", "route_quality", "route_topk",
        "route_counts", "workspace_bytes", "ws_status")

__all__ = list(_API) + ["zha"]


def __getattr__(name):
    if name == "zha" or name in _API:
        import importlib
        mod = importlib.import_module(__name__ + ".zha")
        return mod if name == "zha" else getattr(mod, name)
    raise AttributeError(name)
