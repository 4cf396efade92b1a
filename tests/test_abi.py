"""The C ABI library loads, exports every function include/zha.h declares, and
rejects bad arguments on the host before launching anything (no GPU needed)."""
import ctypes
import math
import os
import re
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zha.h")

zha = pytest.importorskip("hierarchical_kv_cache_amd.zha")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert "zha_route" in names and "dense_attend" in names and len(names) >= 10
    lib = ctypes.CDLL(zha.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(zha.EXPORTS) == names


def test_status_strings_and_workspace_sizes():
    for code in range(7):
        assert zha.status_str(code).startswith("ZHA")
    small = zha.Config(B=1, H_kv=1, G=1, d=64, C=16, L=2, R=4, T_cap=4096)
    big = zha.Config(B=1, H_kv=8, G=4, d=128, C=64, L=3, R=16, T_cap=(1 << 20) + 128)
    assert 0 < zha.workspace_bytes(small) < zha.workspace_bytes(big)
    for op in range(5):
        assert zha.workspace_bytes(big, op) > 0
    assert zha.workspace_bytes(big, zha.OP_ROUTE) <= zha.workspace_bytes(big, zha.OP_ALL)


@pytest.mark.parametrize("bad", [dict(d=96), dict(C=3), dict(C=128), dict(L=9), dict(R=17),
                                 dict(G=0), dict(B=0), dict(kv_dtype=7)])
def test_unsupported_geometry_is_rejected(bad):
    kw = dict(B=1, H_kv=1, G=1, d=64, C=16, L=2, R=4, T_cap=4096)
    kw.update(bad)
    with pytest.raises(zha.ZhaError):
        zha.workspace_bytes(zha.Config(**kw))


def _route(cfg, p=0.9, ws_bytes=None, q=1, leaf=1):
    fake = ctypes.c_void_p(0x1000)
    tree = zha._Tree()
    for i in range(cfg.L):
        tree.khat[i] = 0x2000
        tree.bhat[i] = 0x3000
        tree.n_cap[i] = cfg.level_cap(i + 1)
    tree.n_built = 0x4000
    need = ws_bytes if ws_bytes is not None else zha.workspace_bytes(cfg, zha.OP_ROUTE)
    return zha._lib.zha_route(ctypes.byref(cfg.c()), fake if q else None, ctypes.byref(tree),
                              fake, ctypes.c_float(p), fake if leaf else None, fake, fake,
                              ctypes.c_void_p(0x100000), need,
                              None)


def test_bad_arguments_return_codes_without_launching():
    cfg = zha.Config(B=1, H_kv=2, G=4, d=128, C=64, L=3, R=16, T_cap=1 << 16)
    assert _route(cfg, p=0.0) == zha.EINVAL
    assert _route(cfg, p=1.5) == zha.EINVAL
    assert _route(cfg, p=float("nan")) == zha.EINVAL
    assert _route(cfg, q=0) == zha.EINVAL
    assert _route(cfg, leaf=0) == zha.EINVAL
    assert _route(cfg, ws_bytes=100) == zha.EWORKSPACE
    small_leaf = zha.Config(B=1, H_kv=2, G=4, d=128, C=64, L=3, R=16, T_cap=1 << 16, leaf_cap=10)
    assert _route(small_leaf) == zha.EINVAL
    g17 = zha.Config(B=1, H_kv=1, G=17, d=128, C=64, L=3, R=16, T_cap=1 << 16)
    assert _route(g17, ws_bytes=1 << 30) == zha.EUNSUPPORTED
    out = zha._lib.dense_attend(ctypes.byref(cfg.c()), None, None, None, None, None, 0, None)
    assert out == zha.EINVAL
    fake = ctypes.c_void_p(0x1000)
    tree = zha._Tree()
    for i in range(cfg.L):
        tree.khat[i] = 0x2000
        tree.bhat[i] = 0x3000
        tree.n_cap[i] = cfg.level_cap(i + 1)
    tree.n_built = 0x4000
    need = zha.workspace_bytes(cfg, zha.OP_ROUTE)
    for bad in ([0.9, 1.5, 0.9], [0.9, 0.0, 0.9], [float("nan"), 0.9, 0.9]):
        arr = (ctypes.c_float * 3)(*bad)
        rc = zha._lib.zha_route_sched(ctypes.byref(cfg.c()), fake, ctypes.byref(tree), fake, arr,
                                      fake, fake, fake, ctypes.c_void_p(0x100000), need, None)
        assert rc == zha.EINVAL, bad
    rc = zha._lib.zha_route_sched(ctypes.byref(cfg.c()), fake, ctypes.byref(tree), fake, None,
                                  fake, fake, fake, ctypes.c_void_p(0x100000), need, None)
    assert rc == zha.EINVAL


def test_missing_library_fails_loudly(tmp_path):
    pkg = tmp_path / "hierarchical_kv_cache_amd"
    shutil.copytree(os.path.join(ROOT, "hierarchical_kv_cache_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    code = "import hierarchical_kv_cache_amd as h; h.Config"
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "ImportError" in r.stderr and "not built" in r.stderr


def test_p_schedules_multiply_to_p():
    for L in (1, 3, 6):
        for kind in ("root", "power"):
            pl = zha.p_schedule(kind, 0.8, L, gamma=1.5)
            assert len(pl) == L and all(0 < x <= 1 for x in pl)
            assert abs(math.prod(pl) - 0.8) < 1e-6   # each level rounded to float
        assert zha.p_schedule("uniform", 0.8, L) == [float(np.float32(0.8))] * L
    pw = zha.p_schedule("power", 0.8, 4, gamma=1.0)
    assert pw == sorted(pw)   # the leaf level cuts hardest


@pytest.mark.parametrize("kind", ["uniform", "root", "power"])
def test_p_schedule_matches_the_oracle(kind):
    """zha_p_schedule (host code of the library) against the oracle's float64
    schedule, each level within one float32 step of it."""
    for p in (0.5, 0.75, 0.8, 0.9, 0.99, 1.0):
        pf = float(np.float32(p))
        for L in range(1, zha.MAX_L + 1):
            for gamma in (0.0, 0.5, 1.5, 3.0):
                got = np.array(zha.p_schedule(kind, pf, L, gamma=gamma))
                ref = np.array(O.p_schedule(kind, pf, L, gamma))
                ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
                assert np.all(np.abs(got - ref) <= ulp), (kind, p, L, gamma, got, ref)


def test_p_schedule_rejects_bad_arguments():
    lib = zha._lib
    out = (ctypes.c_float * 8)()
    for kind, p, L, gamma in [(0, 0.9, 0, 1.0), (0, 0.9, zha.MAX_L + 1, 1.0), (1, 0.0, 3, 1.0),
                              (1, 1.5, 3, 1.0), (1, float("nan"), 3, 1.0), (7, 0.9, 3, 1.0),
                              (2, 0.9, 3, float("inf")), (2, 0.9, 3, float("nan"))]:
        assert lib.zha_p_schedule(kind, p, L, gamma, out) == zha.EINVAL, (kind, p, L, gamma)
    assert lib.zha_p_schedule(0, 0.9, 3, 1.0, None) == zha.EINVAL
    with pytest.raises(ValueError):
        zha.p_schedule("cubic", 0.9, 3)


def test_cut_pool_beyond_fixed_point_range_is_rejected():
    """The cut sums masses as w 2^40 in 64 bits: a level-1 pool of 2^24 or more
    entries could wrap, so such a geometry is refused before any launch, while
    the largest pool that fits is accepted."""
    C = 2
    ok = zha.Config(B=1, H_kv=1, G=4, d=64, C=C, L=2, R=4, T_cap=((1 << 24) - 1) * C)
    big = zha.Config(B=1, H_kv=1, G=4, d=64, C=C, L=2, R=4, T_cap=(1 << 24) * C)
    huge_ws = 1 << 40   # sizes are checked, never touched: nothing is launched
    assert _route(big, ws_bytes=huge_ws) == zha.EUNSUPPORTED
    rc = _route(ok, ws_bytes=huge_ws, q=0)   # passes the pool check, fails on the null q
    assert rc == zha.EINVAL
    # zha_route_level: an explicit list longer than the limit
    cfg = zha.Config(B=1, H_kv=1, G=4, d=64, C=C, L=2, R=4, T_cap=(1 << 24) * C + 8,
                     leaf_cap=1 << 25)
    fake = ctypes.c_void_p(0x1000)
    tree = zha._Tree()
    for i in range(cfg.L):
        tree.khat[i] = 0x2000
        tree.bhat[i] = 0x3000
        tree.n_cap[i] = cfg.level_cap(i + 1)
    tree.n_built = 0x4000
    rc = zha._lib.zha_route_level(ctypes.byref(cfg.c()), 1, fake, ctypes.byref(tree), ctypes.c_float(0.9),
                                  fake, fake, fake, 1 << 24, fake, fake, ctypes.c_void_p(0x100000),
                                  huge_ws, None)
    assert rc == zha.EUNSUPPORTED


def test_static_attend_refuses_geometry_beyond_its_scratch():
    """zha_attend_static keeps its scratch in a fixed 64 MiB buffer per device; a
    geometry needing more is refused on the host, before anything is launched
    (16 sequences x 32 query heads at 1M tokens need ~0.5 GB of split partials)."""
    big = zha.Config(B=16, H_kv=8, G=4, d=128, C=64, L=3, R=16, T_cap=1 << 20)
    fake = ctypes.c_void_p(0x1000)
    kv = zha._KV(0x1000, 0x2000, 0x3000)
    rc = zha._lib.zha_attend_static(ctypes.byref(big.c()), fake, ctypes.byref(kv), fake, fake, fake,
                                    fake, fake, None, None)
    assert rc == zha.EWORKSPACE
    rc = zha._lib.zha_attend_static(ctypes.byref(big.c()), None, ctypes.byref(kv), fake, fake, fake,
                                    fake, fake, None, None)
    assert rc == zha.EINVAL


def test_append_needs_its_workspace():
    """The one-launch append keeps per-sequence arrival counters in the workspace:
    a missing or short workspace is refused before any launch."""
    cfg = zha.Config(B=2, H_kv=2, G=4, d=128, C=16, L=2, R=16, T_cap=4096)
    fake = ctypes.c_void_p(0x1000)
    kv = zha._KV(0x1000, 0x2000, 0x3000)
    tree = zha._Tree()
    for i in range(cfg.L):
        tree.khat[i] = 0x2000
        tree.bhat[i] = 0x3000
        tree.n_cap[i] = cfg.level_cap(i + 1)
    tree.n_built = 0x4000
    need = zha.workspace_bytes(cfg, zha.OP_BUILD)
    assert need > 256
    rc = zha._lib.zha_append(ctypes.byref(cfg.c()), ctypes.byref(kv), fake, ctypes.byref(tree), 1,
                             None, 0, None)
    assert rc == zha.EWORKSPACE
    rc = zha._lib.zha_append(ctypes.byref(cfg.c()), ctypes.byref(kv), fake, ctypes.byref(tree), 1,
                             ctypes.c_void_p(0x100000), need - 1, None)
    assert rc == zha.EWORKSPACE
