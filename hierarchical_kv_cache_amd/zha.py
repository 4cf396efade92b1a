"""ctypes binding of libzha (include/zha.h): argument marshalling only.

Every step of tree-summarised decode attention runs in the HIP kernels of
libzha.so; this module passes device pointers of PyTorch tensors and the current
HIP stream, and raises ``ZhaError`` on a non-zero status.  There is no fallback:
if libzha.so is missing the import fails.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import List, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzha.so")

MAX_L = 8
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, ECAPACITY, EHIP, ESTALE = range(7)
F32, BF16 = 0, 1
OP_BUILD, OP_ROUTE, OP_ATTEND, OP_DENSE, OP_ALL = range(5)
SCHED = {"uniform": 0, "root": 1, "power": 2}

EXPORTS = ["zha_workspace_bytes", "zha_status_str", "zha_build_level", "zha_append",
           "zha_route", "zha_route_sched", "zha_route_topk", "zha_route_quality", "zha_route_level", "zha_attend",
           "zha_attend_static", "dense_attend", "zha_route_counts", "zha_ws_status",
           "zha_p_schedule"]


class ZhaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_str(code)} ({code})")


class _Cfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("G", ctypes.c_int32),
                ("d", ctypes.c_int32), ("C", ctypes.c_int32), ("L", ctypes.c_int32),
                ("R", ctypes.c_int32), ("scale", ctypes.c_float), ("rope", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("kv_dtype", ctypes.c_int32),
                ("leaf_cap", ctypes.c_int32), ("T_cap", ctypes.c_int64)]


class _KV(ctypes.Structure):
    _fields_ = [("K", ctypes.c_void_p), ("V", ctypes.c_void_p), ("T", ctypes.c_void_p)]


class _Tree(ctypes.Structure):
    _fields_ = [("khat", ctypes.c_void_p * MAX_L), ("bhat", ctypes.c_void_p * MAX_L),
                ("n_cap", ctypes.c_int64 * MAX_L), ("n_built", ctypes.c_void_p),
                ("khat16", ctypes.c_void_p * MAX_L)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m hierarchical_kv_cache_amd.buildlib`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, f32, i64, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_int64, ctypes.c_size_t
    cfgp, kvp, treep = ctypes.POINTER(_Cfg), ctypes.POINTER(_KV), ctypes.POINTER(_Tree)
    sig = {
        "zha_workspace_bytes": (sz, [cfgp, i32]),
        "zha_status_str": (ctypes.c_char_p, [i32]),
        "zha_build_level": (i32, [cfgp, i32, kvp, P, treep, P, sz, P]),
        "zha_append": (i32, [cfgp, kvp, P, treep, i64, P, sz, P]),
        "zha_route": (i32, [cfgp, P, treep, P, f32, P, P, P, P, sz, P]),
        "zha_route_sched": (i32, [cfgp, P, treep, P, ctypes.POINTER(f32), P, P, P, P, sz, P]),
        "zha_route_topk": (i32, [cfgp, P, treep, P, ctypes.POINTER(i32), P, P, P, P, sz, P]),
        "zha_route_quality": (i32, [cfgp, P, kvp, treep, P, P, sz, P]),
        "zha_route_level": (i32, [cfgp, i32, P, treep, f32, P, P, P, i32, P, P, P, sz, P]),
        "zha_attend": (i32, [cfgp, P, kvp, P, P, P, P, P, P, sz, P]),
        "zha_attend_static": (i32, [cfgp, P, kvp, P, P, P, P, P, P, P]),
        "dense_attend": (i32, [cfgp, P, kvp, P, P, P, sz, P]),
        "zha_route_counts": (i32, [cfgp, P, P, P, P]),
        "zha_ws_status": (i32, [P, P, ctypes.POINTER(i32)]),
        "zha_p_schedule": (i32, [i32, f32, i32, f32, ctypes.POINTER(f32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def status_str(code: int) -> str:
    return _lib.zha_status_str(int(code)).decode()


def _check(code: int, where: str) -> None:
    if code != OK:
        raise ZhaError(code, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libzha must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclasses.dataclass
class Config:
    """Problem geometry (mirrors zha_cfg)."""
    B: int
    H_kv: int
    G: int
    d: int
    C: int
    L: int
    R: int
    T_cap: int
    kv_dtype: int = BF16
    scale: Optional[float] = None
    rope: bool = False
    rope_base: float = 1.0e6
    leaf_cap: Optional[int] = None

    def __post_init__(self):
        if self.scale is None:
            self.scale = 1.0 / math.sqrt(self.d)
        if self.leaf_cap is None:
            self.leaf_cap = max(1, self.T_cap // self.C)

    @property
    def Hq(self) -> int:
        return self.H_kv * self.G

    def c(self) -> _Cfg:
        return _Cfg(self.B, self.H_kv, self.G, self.d, self.C, self.L, self.R,
                    float(self.scale), int(bool(self.rope)), float(self.rope_base),
                    int(self.kv_dtype), int(self.leaf_cap), int(self.T_cap))

    def level_cap(self, level: int) -> int:
        return max(1, self.T_cap // self.C ** level)


def workspace_bytes(cfg: Config, op: int = OP_ALL) -> int:
    n = _lib.zha_workspace_bytes(ctypes.byref(cfg.c()), op)
    if n == 0:
        raise ZhaError(EINVAL, "zha_workspace_bytes")
    return int(n)


def new_workspace(cfg: Config, op: int = OP_ALL, device="cuda") -> torch.Tensor:
    """Zero-filled workspace (the status word must start at zero)."""
    return torch.zeros(workspace_bytes(cfg, op), dtype=torch.uint8, device=device)


class Tree:
    """Device storage of one tree per (sequence, KV head), all levels.

    bf16_copy: also keep a bf16 copy of every level's k_hat (zha_tree.khat16),
    written by the builder and read by the route instead of the fp32 k_hat."""

    def __init__(self, cfg: Config, device="cuda", bf16_copy: bool = False):
        self.cfg = cfg
        self.khat: List[torch.Tensor] = []
        self.bhat: List[torch.Tensor] = []
        for level in range(1, cfg.L + 1):
            n = cfg.level_cap(level)
            self.khat.append(torch.zeros(cfg.B, cfg.H_kv, n, cfg.R, cfg.d, dtype=torch.float32, device=device))
            self.bhat.append(torch.zeros(cfg.B, cfg.H_kv, n, cfg.R, dtype=torch.float32, device=device))
        self.n_built = torch.zeros(cfg.L, cfg.B, dtype=torch.int64, device=device)
        self.khat16: List[Optional[torch.Tensor]] = [None] * cfg.L
        if bf16_copy:
            self.khat16 = [torch.zeros(k.shape, dtype=torch.bfloat16, device=device) for k in self.khat]

    @classmethod
    def lower_levels(cls, tree: "Tree", cfg: "Config") -> "Tree":
        """The lowest cfg.L levels of an existing tree, shared (no copy): for
        example its leaf level alone, as a one-level tree."""
        if cfg.L > tree.cfg.L:
            raise ValueError("the view has more levels than the tree")
        t = cls.__new__(cls)
        t.cfg = cfg
        t.khat = tree.khat[:cfg.L]
        t.bhat = tree.bhat[:cfg.L]
        t.n_built = tree.n_built[:cfg.L]
        t.khat16 = list(getattr(tree, "khat16", [None] * tree.cfg.L))[:cfg.L]
        return t

    def c(self) -> _Tree:
        t = _Tree()
        for i in range(self.cfg.L):
            t.khat[i] = self.khat[i].data_ptr()
            t.bhat[i] = self.bhat[i].data_ptr()
            t.n_cap[i] = self.khat[i].shape[2]
            k16 = getattr(self, "khat16", None)
            if k16 is not None and k16[i] is not None:
                if k16[i].shape != self.khat[i].shape or k16[i].dtype != torch.bfloat16 \
                        or not k16[i].is_contiguous():
                    raise ValueError("khat16 must be a contiguous bf16 tensor shaped like khat")
                t.khat16[i] = k16[i].data_ptr()
        t.n_built = self.n_built.data_ptr()
        return t


def _kv(K, V, T) -> _KV:
    return _KV(K.data_ptr(), V.data_ptr(), T.data_ptr())


def build_level(cfg: Config, level: int, K, V, T, qref, tree: Tree, ws, stream=None):
    _check(_lib.zha_build_level(ctypes.byref(cfg.c()), level, ctypes.byref(_kv(K, V, T)),
                                _ptr(qref), ctypes.byref(tree.c()), _ptr(ws), ws.numel(),
                                _stream(stream)), "zha_build_level")


def build(cfg: Config, K, V, T, qref, tree: Tree, ws, stream=None):
    """All levels, bottom up (prefill)."""
    for level in range(1, cfg.L + 1):
        build_level(cfg, level, K, V, T, qref, tree, ws, stream)


def append(cfg: Config, K, V, T, qref, tree: Tree, ws, max_new_tokens: int = 1, stream=None):
    _check(_lib.zha_append(ctypes.byref(cfg.c()), ctypes.byref(_kv(K, V, T)), _ptr(qref),
                           ctypes.byref(tree.c()), int(max_new_tokens), _ptr(ws), ws.numel(),
                           _stream(stream)), "zha_append")


def route(cfg: Config, q, tree: Tree, T, p, leaf_ids, leaf_mask, leaf_count, ws,
          stream=None):
    """p: one top-p for every level, or a sequence of cfg.L values (entry l-1 for
    level l), which calls zha_route_sched."""
    if isinstance(p, (list, tuple)):
        if len(p) != cfg.L:
            raise ValueError(f"a depth schedule needs {cfg.L} values, got {len(p)}")
        arr = (ctypes.c_float * cfg.L)(*[float(x) for x in p])
        _check(_lib.zha_route_sched(ctypes.byref(cfg.c()), _ptr(q), ctypes.byref(tree.c()),
                                    _ptr(T), arr, _ptr(leaf_ids), _ptr(leaf_mask),
                                    _ptr(leaf_count), _ptr(ws), ws.numel(), _stream(stream)),
               "zha_route_sched")
        return
    _check(_lib.zha_route(ctypes.byref(cfg.c()), _ptr(q), ctypes.byref(tree.c()), _ptr(T),
                          float(p), _ptr(leaf_ids), _ptr(leaf_mask), _ptr(leaf_count),
                          _ptr(ws), ws.numel(), _stream(stream)), "zha_route")


def route_topk(cfg: Config, q, tree: Tree, T, k, leaf_ids, leaf_mask, leaf_count, ws,
               stream=None):
    """Fixed node budget per level: k is one count for every level or cfg.L counts."""
    ks = list(k) if isinstance(k, (list, tuple)) else [int(k)] * cfg.L
    if len(ks) != cfg.L:
        raise ValueError(f"a budget per level needs {cfg.L} values, got {len(ks)}")
    arr = (ctypes.c_int32 * cfg.L)(*[int(x) for x in ks])
    _check(_lib.zha_route_topk(ctypes.byref(cfg.c()), _ptr(q), ctypes.byref(tree.c()), _ptr(T),
                               arr, _ptr(leaf_ids), _ptr(leaf_mask), _ptr(leaf_count), _ptr(ws),
                               ws.numel(), _stream(stream)), "zha_route_topk")


def route_quality(cfg: Config, q, K, V, T, tree: Tree, kl, ws, stream=None):
    """Per-level KL(p || p_hat) of the routing estimate: kl is [L][B][Hq] fp32."""
    _check(_lib.zha_route_quality(ctypes.byref(cfg.c()), _ptr(q), ctypes.byref(_kv(K, V, T)),
                                  ctypes.byref(tree.c()), _ptr(kl), _ptr(ws), ws.numel(),
                                  _stream(stream)), "zha_route_quality")


def p_schedule(kind: str, p: float, L: int, gamma: float = 1.0) -> List[float]:
    """Per-level top-p of a depth schedule (zha_p_schedule; entry l-1 for level
    l): "uniform" (p at every level), "root" (p^(1/L)) or "power" (p^(w_l),
    w_l proportional to l^-gamma and summing to one)."""
    if kind not in SCHED:
        raise ValueError(f"unknown schedule {kind!r}")
    arr = (ctypes.c_float * max(1, int(L)))()
    _check(_lib.zha_p_schedule(SCHED[kind], float(p), int(L), float(gamma), arr), "zha_p_schedule")
    return [float(x) for x in arr[:L]]


def route_level(cfg: Config, level: int, q, tree: Tree, p: float, cand_ids, cand_mask,
                cand_count, scores, sel, ws, stream=None):
    cap = cand_ids.shape[-1]
    _check(_lib.zha_route_level(ctypes.byref(cfg.c()), level, _ptr(q), ctypes.byref(tree.c()),
                                float(p), _ptr(cand_ids), _ptr(cand_mask), _ptr(cand_count),
                                int(cap), _ptr(scores), _ptr(sel), _ptr(ws), ws.numel(),
                                _stream(stream)), "zha_route_level")


def attend(cfg: Config, q, K, V, T, leaf_ids, leaf_mask, leaf_count, out, lse, ws, stream=None):
    _check(_lib.zha_attend(ctypes.byref(cfg.c()), _ptr(q), ctypes.byref(_kv(K, V, T)),
                           _ptr(leaf_ids), _ptr(leaf_mask), _ptr(leaf_count), _ptr(out),
                           _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)), "zha_attend")


def attend_static(cfg: Config, q, K, V, T, leaf_ids, leaf_mask, leaf_count, out, lse,
                  status=None, stream=None):
    """zha_attend with the library's own per-device scratch (no workspace; nothing
    allocated).  status: optional int32 device tensor for device-detected errors."""
    _check(_lib.zha_attend_static(ctypes.byref(cfg.c()), _ptr(q), ctypes.byref(_kv(K, V, T)),
                                  _ptr(leaf_ids), _ptr(leaf_mask), _ptr(leaf_count), _ptr(out),
                                  _ptr(lse), _ptr(status), _stream(stream)), "zha_attend_static")


def dense_attend(cfg: Config, q, K, V, T, out, lse, ws, stream=None):
    _check(_lib.dense_attend(ctypes.byref(cfg.c()), _ptr(q), ctypes.byref(_kv(K, V, T)),
                             _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)),
           "dense_attend")


def route_counts(cfg: Config, ws, union_count, kept_count, stream=None):
    """Per-level candidate-union sizes [L][B][H_kv] and kept counts [L][B][Hq] of
    the last route on ``ws`` (int32 device tensors, filled asynchronously)."""
    _check(_lib.zha_route_counts(ctypes.byref(cfg.c()), _ptr(ws), _ptr(union_count),
                                 _ptr(kept_count), _stream(stream)), "zha_route_counts")


def ws_status(ws, stream=None) -> int:
    st = ctypes.c_int32(0)
    _check(_lib.zha_ws_status(_ptr(ws), _stream(stream), ctypes.byref(st)), "zha_ws_status")
    return int(st.value)


class LeafList:
    """Route output / attend input buffers for one config."""

    def __init__(self, cfg: Config, device="cuda"):
        self.ids = torch.zeros(cfg.B, cfg.H_kv, cfg.leaf_cap, dtype=torch.int32, device=device)
        self.mask = torch.zeros(cfg.B, cfg.H_kv, cfg.leaf_cap, dtype=torch.int32, device=device)
        self.count = torch.zeros(cfg.B, cfg.H_kv, dtype=torch.int32, device=device)


class Decoder:
    """One decode step of tree-summarised attention: (append) -> route -> attend.

    Holds the tree, the workspace and the leaf list; the caller owns K, V, T and
    writes each new token's key/value before the step, as a KV cache does.
    bf16_copy: the tree also keeps a bf16 copy of every level's k_hat, which the
    builder writes and the route scores from (half the summary bytes per step).
    """

    def __init__(self, cfg: Config, qref: torch.Tensor, device="cuda", bf16_copy: bool = False):
        self.cfg = cfg
        self.qref = qref
        self.tree = Tree(cfg, device, bf16_copy)
        self.ws = new_workspace(cfg, OP_ALL, device)
        self.leaves = LeafList(cfg, device)
        self.out = torch.zeros(cfg.B, cfg.Hq, cfg.d, dtype=torch.float32, device=device)
        self.lse = torch.zeros(cfg.B, cfg.Hq, dtype=torch.float32, device=device)

    def prefill(self, K, V, T):
        build(self.cfg, K, V, T, self.qref, self.tree, self.ws)

    def append(self, K, V, T, max_new_tokens: int = 1):
        append(self.cfg, K, V, T, self.qref, self.tree, self.ws, max_new_tokens)

    def step(self, q, K, V, T, p: float):
        route(self.cfg, q, self.tree, T, p, self.leaves.ids, self.leaves.mask,
              self.leaves.count, self.ws)
        attend(self.cfg, q, K, V, T, self.leaves.ids, self.leaves.mask, self.leaves.count,
               self.out, self.lse, self.ws)
        return self.out, self.lse

    def dense(self, q, K, V, T):
        dense_attend(self.cfg, q, K, V, T, self.out, self.lse, self.ws)
        return self.out, self.lse
