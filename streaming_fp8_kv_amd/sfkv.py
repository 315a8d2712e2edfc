"""ctypes binding of libsfkv.so (the C ABI in include/sfkv.h).

Argument marshalling only: every step of the cache path runs in the HIP
kernels behind the C ABI. PyTorch provides device memory and the current HIP
stream. The module raises on import when the library has not been built; there
is no fallback implementation.

The function names mirror the C entry points without their ``sfkv_`` prefix:
``rope_bytes``, ``rope_init``, ``cache_bytes``, ``cache_init``,
``calibrate_scales``, ``cache_write``, ``attend_workspace_bytes``, ``attend``,
``write_attend``, ``write_attend_noalloc``, ``rebase_positions``,
``rebase_positions_many``, ``cache_state``, ``cache_layout``, and for the launch
software's plain linear window ``linear_bytes``, ``linear_init``,
``linear_calibrate_scales``, ``linear_write``, ``linear_workspace_bytes``,
``linear_attend``, ``linear_state``, ``linear_layout``. ``Rope``,
``RingCache`` and ``LinearCache`` bundle a handle with the torch buffer it
lives in.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsfkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with `python -m streaming_fp8_kv_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

OK, EINVAL, ESTATE, ERANGE, EHIP = 0, -1, -2, -3, -4
BF16, FP32 = 0, 1

# every symbol include/sfkv.h declares
SYMBOLS = (
    "sfkv_rope_bytes", "sfkv_rope_init", "sfkv_rope_destroy",
    "sfkv_cache_bytes", "sfkv_cache_init", "sfkv_cache_destroy",
    "sfkv_calibrate_scales", "sfkv_cache_write",
    "sfkv_attend_workspace_bytes", "sfkv_attend", "sfkv_write_attend", "sfkv_rebase_positions",
    "sfkv_rebase_positions_many", "sfkv_write_attend_noalloc",
    "sfkv_cache_state", "sfkv_cache_layout",
    "sfkv_linear_bytes", "sfkv_linear_init", "sfkv_linear_destroy",
    "sfkv_linear_calibrate_scales", "sfkv_linear_write", "sfkv_linear_workspace_bytes",
    "sfkv_linear_attend", "sfkv_linear_state", "sfkv_linear_layout",
    "sfkv_status_string", "sfkv_last_error",
)


STORE_E4M3, STORE_BF16 = 0, 1       # sfkv_storage


class CacheConfig(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("max_new_tokens", ctypes.c_int32),
                ("storage", ctypes.c_int32)]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_P = ctypes.POINTER


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("sfkv_rope_bytes", _sz, _i32, _i32)
_sig("sfkv_rope_init", ctypes.c_int, ctypes.c_double, _i32, _i32, _vp, _sz, _vp, _P(_vp))
_sig("sfkv_rope_destroy", None, _vp)
_sig("sfkv_cache_bytes", _sz, _P(CacheConfig))
_sig("sfkv_cache_init", ctypes.c_int, _P(CacheConfig), _vp, _vp, _sz, _vp, _P(_vp))
_sig("sfkv_cache_destroy", None, _vp)
_sig("sfkv_calibrate_scales", ctypes.c_int, _vp, _vp, _vp, ctypes.c_int, _i32, _vp)
_sig("sfkv_cache_write", ctypes.c_int, _vp, _vp, _vp, ctypes.c_int, _i32, _vp)
_sig("sfkv_attend_workspace_bytes", _sz, _vp)
_sig("sfkv_attend", ctypes.c_int, _vp, _vp, ctypes.c_int, _i32, _vp, _vp, _sz, _vp)
_sig("sfkv_write_attend", ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _vp, _vp, _sz, _vp)
_sig("sfkv_write_attend_noalloc", ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _vp, _vp)
_sig("sfkv_rebase_positions", ctypes.c_int, _vp, _i64, _vp)
_sig("sfkv_rebase_positions_many", ctypes.c_int, _P(_vp), _P(_i64), _i32, _vp)
_sig("sfkv_cache_state", ctypes.c_int, _vp, _P(_i64), _P(_i64), _P(_i32), _P(_i32))
_sig("sfkv_cache_layout", ctypes.c_int, _vp, _P(_sz), _P(_sz), _P(_sz), _P(_sz))
_sig("sfkv_linear_bytes", _sz, _P(CacheConfig), ctypes.c_int)
_sig("sfkv_linear_init", ctypes.c_int, _P(CacheConfig), _vp, ctypes.c_int, _vp, _sz, _vp, _P(_vp))
_sig("sfkv_linear_destroy", None, _vp)
_sig("sfkv_linear_calibrate_scales", ctypes.c_int, _vp, _vp, _vp, _i32, _vp)
_sig("sfkv_linear_write", ctypes.c_int, _vp, _vp, _vp, _i32, _vp)
_sig("sfkv_linear_workspace_bytes", _sz, _vp)
_sig("sfkv_linear_attend", ctypes.c_int, _vp, _vp, _i32, _vp, _vp, _sz, _vp)
_sig("sfkv_linear_state", ctypes.c_int, _vp, _P(_i32), _P(_i32))
_sig("sfkv_linear_layout", ctypes.c_int, _vp, _P(_sz), _P(_sz), _P(_sz), _P(_sz))
_sig("sfkv_status_string", ctypes.c_char_p, ctypes.c_int)
_sig("sfkv_last_error", ctypes.c_char_p)


class SfkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_lib.sfkv_status_string(status).decode()} ({status}): {message}")
        self.status = status


def _check(status: int):
    if status != OK:
        raise SfkvError(status, _lib.sfkv_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError("inputs must be bfloat16 or float32")


def _frame(t: torch.Tensor, heads: int, head_dim: int) -> torch.Tensor:
    if not t.is_cuda or not t.is_contiguous() or t.dim() != 3 or tuple(t.shape[1:]) != (heads, head_dim):
        raise ValueError("expected a contiguous CUDA tensor of shape [n, heads, head_dim]")
    return t


# The library sees only pointers: it reads every input with the first one's
# dtype and row count and writes n_q * heads * head_dim floats to out, so the
# binding refuses tensors that would let a kernel read or write past an end.
def _device_buf(t: torch.Tensor, what: str) -> torch.Tensor:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous CUDA tensor")
    return t


def _same_frame(first: torch.Tensor, *others: torch.Tensor):
    for t in (first,) + others:
        _device_buf(t, "every input")
        if t.dim() != 3:
            raise ValueError("inputs must have shape [n, heads, head_dim]")
    for t in others:
        if t.dtype != first.dtype or t.shape != first.shape or t.device != first.device:
            raise ValueError("inputs of one call must share one dtype, shape [n, heads, head_dim] and device")


def _out_for(out: torch.Tensor, q: torch.Tensor):
    _device_buf(out, "out")
    if out.dtype != torch.float32 or out.shape != q.shape or out.device != q.device:
        raise ValueError("out must be a float32 tensor of q's shape on q's device")


def _workspace(ws: Optional[torch.Tensor], q: torch.Tensor):
    if ws is None:
        return None, 0
    _device_buf(ws, "workspace")
    if ws.device != q.device:
        raise ValueError("workspace must be on q's device")
    return ws.data_ptr(), ws.numel() * ws.element_size()


# ---- C entry points -----------------------------------------------------------
def rope_bytes(head_dim: int, max_position: int) -> int:
    return int(_lib.sfkv_rope_bytes(head_dim, max_position))


def rope_init(base: float, head_dim: int, max_position: int, buf: torch.Tensor, stream=None) -> int:
    h = _vp()
    _device_buf(buf, "buf")
    _check(_lib.sfkv_rope_init(base, head_dim, max_position, buf.data_ptr(), buf.numel(),
                               _stream(stream), ctypes.byref(h)))
    return h.value


def cache_bytes(cfg: CacheConfig) -> int:
    return int(_lib.sfkv_cache_bytes(ctypes.byref(cfg)))


def cache_init(cfg: CacheConfig, rope_handle: int, buf: torch.Tensor, stream=None) -> int:
    h = _vp()
    _device_buf(buf, "buf")
    _check(_lib.sfkv_cache_init(ctypes.byref(cfg), rope_handle, buf.data_ptr(), buf.numel(),
                                _stream(stream), ctypes.byref(h)))
    return h.value


def calibrate_scales(handle: int, k: torch.Tensor, v: torch.Tensor, stream=None):
    _same_frame(k, v)
    _check(_lib.sfkv_calibrate_scales(handle, k.data_ptr(), v.data_ptr(), _dtype_code(k),
                                      k.shape[0], _stream(stream)))


def cache_write(handle: int, k: torch.Tensor, v: torch.Tensor, stream=None):
    _same_frame(k, v)
    _check(_lib.sfkv_cache_write(handle, k.data_ptr(), v.data_ptr(), _dtype_code(k),
                                 k.shape[0], _stream(stream)))


def attend_workspace_bytes(handle: int) -> int:
    return int(_lib.sfkv_attend_workspace_bytes(handle))


def attend(handle: int, q: torch.Tensor, out: torch.Tensor, workspace: Optional[torch.Tensor] = None,
           stream=None):
    _same_frame(q)
    _out_for(out, q)
    ws_ptr, ws_len = _workspace(workspace, q)
    _check(_lib.sfkv_attend(handle, q.data_ptr(), _dtype_code(q), q.shape[0], out.data_ptr(),
                            ws_ptr, ws_len, _stream(stream)))


def write_attend(handle: int, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    code = _dtype_code(k)
    _same_frame(k, v, q)
    _out_for(out, q)
    ws_ptr, ws_len = _workspace(workspace, q)
    _check(_lib.sfkv_write_attend(handle, k.data_ptr(), v.data_ptr(), q.data_ptr(), code, k.shape[0],
                                  out.data_ptr(), ws_ptr, ws_len, _stream(stream)))


def write_attend_noalloc(handle: int, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                         stream=None):
    """write_attend with the library's static scratch instead of a workspace."""
    code = _dtype_code(k)
    _same_frame(k, v, q)
    _out_for(out, q)
    _check(_lib.sfkv_write_attend_noalloc(handle, k.data_ptr(), v.data_ptr(), q.data_ptr(), code, k.shape[0],
                                          out.data_ptr(), _stream(stream)))


def rebase_positions(handle: int, delta: int, stream=None):
    _check(_lib.sfkv_rebase_positions(handle, int(delta), _stream(stream)))


def rebase_positions_many(handles, deltas, stream=None):
    """One delta rotation per cache: handles[i] by deltas[i], as few launches."""
    handles, deltas = list(handles), [int(d) for d in deltas]
    if len(handles) != len(deltas):
        raise ValueError("one delta per cache")
    hs = (_vp * len(handles))(*handles)
    ds = (_i64 * len(deltas))(*deltas)
    _check(_lib.sfkv_rebase_positions_many(hs, ds, len(handles), _stream(stream)))


def cache_state(handle: int) -> dict:
    t, p, s, n = _i64(), _i64(), _i32(), _i32()
    _check(_lib.sfkv_cache_state(handle, ctypes.byref(t), ctypes.byref(p), ctypes.byref(s), ctypes.byref(n)))
    return {"tokens": t.value, "next_pos": p.value, "write_slot": s.value, "n_valid": n.value}


def cache_layout(handle: int) -> dict:
    k, v, p, s = _sz(), _sz(), _sz(), _sz()
    _check(_lib.sfkv_cache_layout(handle, ctypes.byref(k), ctypes.byref(v), ctypes.byref(p), ctypes.byref(s)))
    return {"k": k.value, "v": v.value, "pos": p.value, "scales": s.value}


def linear_bytes(cfg: CacheConfig, dtype: int) -> int:
    return int(_lib.sfkv_linear_bytes(ctypes.byref(cfg), dtype))


def linear_init(cfg: CacheConfig, rope_handle: int, dtype: int, buf: torch.Tensor, stream=None) -> int:
    h = _vp()
    _device_buf(buf, "buf")
    _check(_lib.sfkv_linear_init(ctypes.byref(cfg), rope_handle, dtype, buf.data_ptr(), buf.numel(),
                                 _stream(stream), ctypes.byref(h)))
    return h.value


def linear_calibrate_scales(handle: int, k: torch.Tensor, v: torch.Tensor, stream=None):
    _same_frame(k, v)
    _check(_lib.sfkv_linear_calibrate_scales(handle, k.data_ptr(), v.data_ptr(), k.shape[0], _stream(stream)))


def linear_write(handle: int, k: torch.Tensor, v: torch.Tensor, stream=None):
    _same_frame(k, v)
    _check(_lib.sfkv_linear_write(handle, k.data_ptr(), v.data_ptr(), k.shape[0], _stream(stream)))


def linear_workspace_bytes(handle: int) -> int:
    return int(_lib.sfkv_linear_workspace_bytes(handle))


def linear_attend(handle: int, q: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor, stream=None):
    _same_frame(q)
    _out_for(out, q)
    ws_ptr, ws_len = _workspace(workspace, q)
    _check(_lib.sfkv_linear_attend(handle, q.data_ptr(), q.shape[0], out.data_ptr(), ws_ptr, ws_len,
                                   _stream(stream)))


def linear_state(handle: int) -> dict:
    m, n = _i32(), _i32()
    _check(_lib.sfkv_linear_state(handle, ctypes.byref(m), ctypes.byref(n)))
    return {"n_window": m.value, "last_n": n.value}


def linear_layout(handle: int) -> dict:
    k, v, p, s = _sz(), _sz(), _sz(), _sz()
    _check(_lib.sfkv_linear_layout(handle, ctypes.byref(k), ctypes.byref(v), ctypes.byref(p), ctypes.byref(s)))
    return {"k": k.value, "v": v.value, "pos": p.value, "scales": s.value}


# ---- owners -------------------------------------------------------------------
class Rope:
    """RoPE table in a torch device buffer, shared by every cache of one head_dim."""

    def __init__(self, head_dim: int, max_position: int = 65536, base: float = 10000.0,
                 device="cuda", stream=None):
        self.head_dim, self.max_position, self.base = head_dim, max_position, base
        n = rope_bytes(head_dim, max_position)
        if n == 0:
            raise ValueError("invalid head_dim or max_position")
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        self._destroy = _lib.sfkv_rope_destroy     # still reachable at interpreter exit
        self.handle = rope_init(base, head_dim, max_position, self.buf, stream)

    def __del__(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None


class RingCache:
    """One ring cache: its device buffer, handle and views of its contents."""

    def __init__(self, rope: Rope, heads: int, capacity: int, max_new_tokens: Optional[int] = None,
                 device="cuda", stream=None, storage: int = STORE_E4M3):
        self.rope = rope
        self.cfg = CacheConfig(heads, rope.head_dim, capacity, max_new_tokens or capacity, storage)
        n = cache_bytes(self.cfg)
        if n == 0:
            raise ValueError("invalid cache configuration")
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        self._destroy = _lib.sfkv_cache_destroy    # still reachable at interpreter exit
        self.handle = cache_init(self.cfg, rope.handle, self.buf, stream)
        self.layout = cache_layout(self.handle)

    def __del__(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None

    # compute calls
    def calibrate_scales(self, k, v, stream=None):
        calibrate_scales(self.handle, _frame(k, self.cfg.num_heads, self.cfg.head_dim),
                         _frame(v, self.cfg.num_heads, self.cfg.head_dim), stream)

    def cache_write(self, k, v, stream=None):
        cache_write(self.handle, _frame(k, self.cfg.num_heads, self.cfg.head_dim),
                    _frame(v, self.cfg.num_heads, self.cfg.head_dim), stream)

    def workspace_bytes(self) -> int:
        return attend_workspace_bytes(self.handle)

    def attend(self, q, out=None, workspace=None, stream=None):
        q = _frame(q, self.cfg.num_heads, self.cfg.head_dim)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = torch.empty(self.workspace_bytes(), dtype=torch.uint8, device=q.device)
        attend(self.handle, q, out, workspace, stream)
        return out

    def write_attend(self, k, v, q, out=None, workspace=None, stream=None):
        """cache_write(k, v) then attend(q) in one call (one launch fewer)."""
        H, d = self.cfg.num_heads, self.cfg.head_dim
        k, v, q = _frame(k, H, d), _frame(v, H, d), _frame(q, H, d)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = torch.empty(self.workspace_bytes(), dtype=torch.uint8, device=q.device)
        write_attend(self.handle, k, v, q, out, workspace, stream)
        return out

    def rebase_positions(self, delta: int, stream=None):
        rebase_positions(self.handle, delta, stream)

    def state(self) -> dict:
        return cache_state(self.handle)

    # views into the device buffer (no copies); codes are uint8 E4M3 bytes or,
    # with bf16 storage, int16 views of the bfloat16 bit patterns
    def _plane(self, key: str) -> torch.Tensor:
        c = self.cfg
        es = 2 if c.storage == STORE_BF16 else 1
        n = c.num_heads * c.capacity * c.head_dim * es
        t = self.buf[self.layout[key]:self.layout[key] + n]
        if es == 2:
            t = t.view(torch.int16)
        return t.view(c.num_heads, c.capacity, c.head_dim)

    def k_codes(self) -> torch.Tensor:
        return self._plane("k")

    def v_codes(self) -> torch.Tensor:
        return self._plane("v")

    def positions(self) -> torch.Tensor:
        c = self.cfg
        return self.buf[self.layout["pos"]:self.layout["pos"] + 4 * c.capacity].view(torch.int32)

    def scales(self) -> torch.Tensor:
        c = self.cfg
        return self.buf[self.layout["scales"]:self.layout["scales"] + 16 * c.num_heads].view(torch.float32).view(4, c.num_heads)


class LinearCache:
    """The launch software's plain path: a copy-shifted raw window re-rotated and
    re-quantised on every write (its device buffer, handle and views)."""

    def __init__(self, rope: Rope, heads: int, capacity: int, max_new_tokens: Optional[int] = None,
                 dtype: torch.dtype = torch.bfloat16, device="cuda", stream=None):
        self.rope = rope
        self.dtype = dtype
        self.code = BF16 if dtype == torch.bfloat16 else FP32
        if dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("dtype must be bfloat16 or float32")
        self.cfg = CacheConfig(heads, rope.head_dim, capacity, max_new_tokens or capacity)
        n = linear_bytes(self.cfg, self.code)
        if n == 0:
            raise ValueError("invalid cache configuration")
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        self._destroy = _lib.sfkv_linear_destroy    # still reachable at interpreter exit
        self.handle = linear_init(self.cfg, rope.handle, self.code, self.buf, stream)
        self.layout = linear_layout(self.handle)

    def __del__(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None

    def _in(self, t):
        t = _frame(t, self.cfg.num_heads, self.cfg.head_dim)
        if t.dtype != self.dtype:
            raise TypeError(f"expected {self.dtype} inputs for this window")
        return t

    def calibrate_scales(self, k, v, stream=None):
        linear_calibrate_scales(self.handle, self._in(k), self._in(v), stream)

    def cache_write(self, k, v, stream=None):
        linear_write(self.handle, self._in(k), self._in(v), stream)

    def workspace_bytes(self) -> int:
        return linear_workspace_bytes(self.handle)

    def attend(self, q, out=None, workspace=None, stream=None):
        q = self._in(q)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = torch.empty(self.workspace_bytes(), dtype=torch.uint8, device=q.device)
        linear_attend(self.handle, q, out, workspace, stream)
        return out

    def state(self) -> dict:
        return linear_state(self.handle)

    def k_codes(self) -> torch.Tensor:
        c = self.cfg
        n = c.num_heads * c.capacity * c.head_dim
        return self.buf[self.layout["k"]:self.layout["k"] + n].view(c.num_heads, c.capacity, c.head_dim)

    def v_codes(self) -> torch.Tensor:
        c = self.cfg
        n = c.num_heads * c.capacity * c.head_dim
        return self.buf[self.layout["v"]:self.layout["v"] + n].view(c.num_heads, c.capacity, c.head_dim)

    def positions(self) -> torch.Tensor:
        c = self.cfg
        return self.buf[self.layout["pos"]:self.layout["pos"] + 4 * c.capacity].view(torch.int32)

    def scales(self) -> torch.Tensor:
        c = self.cfg
        return self.buf[self.layout["scales"]:self.layout["scales"] + 16 * c.num_heads].view(torch.float32).view(4, c.num_heads)
