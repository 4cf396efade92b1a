"""The library's host code under AddressSanitizer (CPU only, no GPU needed).

libzha is rebuilt with ASan on its host code alone (the device code is compiled
as usual and never runs here), and the ABI tests -- argument checks, workspace
sizing, depth schedules, rejection of bad geometries -- run against it in a
child process with the ASan runtime preloaded.  A deliberate heap overflow
through the ABI first shows that the sanitizer is live in that setup.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hierarchical_kv_cache_amd", "csrc")
SOURCES = ["api.hip", "attend.hip", "build.hip", "route.hip"]
# host-side instrumentation only: every sanitizer flag goes to the host pass
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _asan_runtime():
    pats = ["/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
            "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"]
    for pat in pats:
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    return None


def _build(tmp):
    cc = _hipcc()
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wno-unused-result", *HOST_ASAN]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(tmp, src.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p, src in zip(procs, SOURCES):
        _, err = p.communicate()
        assert p.returncode == 0, f"hipcc failed on {src}:\n{err}"
    pkg = os.path.join(tmp, "hierarchical_kv_cache_amd")
    os.makedirs(pkg)
    for f in glob.glob(os.path.join(ROOT, "hierarchical_kv_cache_amd", "*.py")):
        shutil.copy(f, pkg)
    r = subprocess.run([cc, "-shared", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        "-o", os.path.join(pkg, "libzha.so"), *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    for d in ("include", "oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(tmp, d),
                        ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp)


@pytest.mark.skipif(_hipcc() is None or _asan_runtime() is None,
                    reason="needs hipcc and the clang ASan runtime")
def test_abi_host_code_under_asan(tmp_path):
    tmp = str(tmp_path)
    _build(tmp)
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               PYTHONDONTWRITEBYTECODE="1")
    # the sanitizer is live: a 3-level schedule written into a 1-float heap array
    probe = ("import ctypes\n"
             "from hierarchical_kv_cache_amd import zha\n"
             "libc = ctypes.CDLL(None)\n"
             "libc.malloc.restype = ctypes.c_void_p\n"
             "buf = libc.malloc(4)\n"
             "zha._lib.zha_p_schedule(1, 0.9, 3, 1.0, ctypes.cast(buf, ctypes.POINTER(ctypes.c_float)))\n")
    r = subprocess.run([sys.executable, "-c", probe], cwd=tmp, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.returncode, r.stderr[-2000:])
    # the ABI tests, clean under the sanitizer
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "AddressSanitizer" not in out, out[-4000:]
