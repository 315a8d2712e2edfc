"""The C-ABI library on the host: it loads, exports every declared symbol, sizes
its buffers as documented, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sfkv.h")


@pytest.fixture(scope="module")
def sfkv():
    from streaming_fp8_kv_amd import sfkv as lib
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sfkv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for call in ("sfkv_cache_init", "sfkv_calibrate_scales", "sfkv_cache_write",
                 "sfkv_attend", "sfkv_rebase_positions"):
        assert call in names


def test_every_declared_symbol_is_exported(sfkv):
    names = declared_functions()
    assert set(names) == set(sfkv.SYMBOLS)
    lib = ctypes.CDLL(sfkv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_buffer_sizes(sfkv):
    cfg = sfkv.CacheConfig(24, 128, 5788, 757)
    plane = 24 * 5788 * 128
    n = sfkv.cache_bytes(cfg)
    assert n % 256 == 0
    assert n >= 2 * plane + 4 * 5788 + 16 * 24
    assert n < 2 * plane + 4 * 5788 + 16 * 24 + 4 * 256
    assert sfkv.rope_bytes(128, 65536) == 65537 * 64 * 8
    assert sfkv.rope_bytes(64, 1024) == 1025 * 32 * 8


def test_bf16_storage_sizes(sfkv):
    # bf16 storage: two bytes per element in both planes, same positions and
    # scale slots; the plane-size limit counts bytes, so it halves in tokens
    cfg = sfkv.CacheConfig(24, 128, 5788, 757, sfkv.STORE_BF16)
    plane = 2 * 24 * 5788 * 128
    n = sfkv.cache_bytes(cfg)
    assert n % 256 == 0
    assert 2 * plane + 4 * 5788 + 16 * 24 <= n < 2 * plane + 4 * 5788 + 16 * 24 + 4 * 256
    assert sfkv.cache_bytes(sfkv.CacheConfig(64, 128, 1 << 17, 16, sfkv.STORE_E4M3)) > 0   # 2^30 B
    assert sfkv.cache_bytes(sfkv.CacheConfig(64, 128, 1 << 17, 16, sfkv.STORE_BF16)) == 0  # 2^31 B
    for bad in (2, -1, 7):
        assert sfkv.cache_bytes(sfkv.CacheConfig(24, 128, 5788, 757, bad)) == 0
    # the plain linear window keeps E4M3 storage only
    assert sfkv.linear_bytes(cfg, sfkv.BF16) == 0


def test_linear_buffer_sizes(sfkv):
    cfg = sfkv.CacheConfig(24, 128, 5788, 757)
    planes = sfkv.cache_bytes(cfg)
    window = 5788 * 24 * 128
    for code, esize in ((sfkv.BF16, 2), (sfkv.FP32, 4)):
        n = sfkv.linear_bytes(cfg, code)
        assert n % 256 == 0
        assert planes + 4 * window * esize <= n < planes + 4 * window * esize + 2 * 256
    assert sfkv.linear_bytes(cfg, 7) == 0
    assert sfkv.linear_bytes(sfkv.CacheConfig(1, 96, 64, 16), sfkv.BF16) == 0


@pytest.mark.parametrize("cfg", [
    (0, 128, 64, 16), (1, 96, 64, 16), (1, 128, 0, 1), (1, 128, 64, 0), (1, 128, 64, 65),
    (4096, 128, 1 << 24, 16),     # a code plane of 2^43 bytes
])
def test_bad_configs_size_zero_and_fail_init(sfkv, cfg):
    c = sfkv.CacheConfig(*cfg)
    assert sfkv.cache_bytes(c) == 0
    h = ctypes.c_void_p()
    st = sfkv._lib.sfkv_cache_init(ctypes.byref(c), None, None, 0, None, ctypes.byref(h))
    assert st == sfkv.EINVAL and not h.value
    assert sfkv._lib.sfkv_last_error()


@pytest.mark.parametrize("base,d,maxp,ptr,nbytes", [
    (10000.0, 96, 100, 256, 1 << 20),       # head_dim
    (10000.0, 128, 0, 256, 1 << 20),        # max_position
    (1.0, 128, 100, 256, 1 << 20),          # base
    (float("inf"), 128, 100, 256, 1 << 20),
    (10000.0, 128, 100, 0, 1 << 20),        # NULL memory
    (10000.0, 128, 100, 258, 1 << 20),      # misaligned
    (10000.0, 128, 100, 256, 100),          # too small
])
def test_rope_init_validation(sfkv, base, d, maxp, ptr, nbytes):
    h = ctypes.c_void_p()
    st = sfkv._lib.sfkv_rope_init(base, d, maxp, ptr or None, nbytes, None, ctypes.byref(h))
    assert st == sfkv.EINVAL and not h.value


def test_null_handles(sfkv):
    lib = sfkv._lib
    assert lib.sfkv_cache_write(None, 256, 256, 0, 1, None) == sfkv.EINVAL
    assert lib.sfkv_calibrate_scales(None, 256, 256, 0, 1, None) == sfkv.EINVAL
    assert lib.sfkv_attend(None, 256, 0, 1, 256, None, 0, None) == sfkv.EINVAL
    assert lib.sfkv_write_attend(None, 256, 256, 256, 0, 1, 256, None, 0, None) == sfkv.EINVAL
    assert lib.sfkv_rebase_positions(None, 0, None) == sfkv.EINVAL
    assert lib.sfkv_rebase_positions_many(None, None, 0, None) == sfkv.OK
    assert lib.sfkv_rebase_positions_many(None, None, 1, None) == sfkv.EINVAL
    assert lib.sfkv_rebase_positions_many(None, None, -1, None) == sfkv.EINVAL
    nulls = (ctypes.c_void_p * 2)(None, None)
    zeros = (ctypes.c_int64 * 2)(0, 0)
    assert lib.sfkv_rebase_positions_many(nulls, zeros, 2, None) == sfkv.EINVAL
    assert lib.sfkv_cache_state(None, None, None, None, None) == sfkv.EINVAL
    assert lib.sfkv_attend_workspace_bytes(None) == 0
    assert lib.sfkv_linear_write(None, 256, 256, 1, None) == sfkv.EINVAL
    assert lib.sfkv_linear_calibrate_scales(None, 256, 256, 1, None) == sfkv.EINVAL
    assert lib.sfkv_linear_attend(None, 256, 1, 256, None, 0, None) == sfkv.EINVAL
    assert lib.sfkv_linear_state(None, None, None) == sfkv.EINVAL
    assert lib.sfkv_linear_workspace_bytes(None) == 0
    assert lib.sfkv_status_string(-3) == b"position out of range"


def test_binding_has_no_fallback():
    src = open(os.path.join(ROOT, "streaming_fp8_kv_amd", "sfkv.py")).read()
    assert "import oracle" not in src and "from oracle" not in src
    assert "raise ImportError" in src


def test_c_session_usage():
    """The C consumer of the ABI links against the library and rejects a bad
    command line before touching the GPU."""
    import subprocess
    exe = os.path.join(ROOT, "tests", "c_abi", "session")
    if not os.path.exists(exe):
        pytest.skip("tests/c_abi/session not built")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
