"""Python binding of libtwnorm: fused reduce of N tensor-parallel partials +
residual add + RMSNorm * weight on one MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libtwnorm.so`` (built in-tree by ``reduce_residual_add_amd.build``).
PyTorch provides device memory and the current HIP stream.  There is no CPU
fallback: if the library is missing, every call raises.

The C entry points are declared in ``include/twnorm.h`` (the measurement and
tuning aids in ``include/twnorm_bench.h``); the functions below carry the same
names without the ``tw_`` prefix.
"""
from __future__ import annotations

import atexit
import ctypes
import os
from typing import Optional, Sequence

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libtwnorm.so")

TW_OK, TW_ERR_INVALID_ARG, TW_ERR_UNSUPPORTED, TW_ERR_ALIAS, TW_ERR_HIP = 0, -1, -2, -3, -4
TW_BF16, TW_F32 = 0, 1
TW_MAX_PARTIALS = 16
TW_ABI_VERSION = 4

_lib: Optional[ctypes.CDLL] = None

_c = ctypes
_vp = _c.c_void_p
_i64 = _c.c_int64


class TwError(RuntimeError):
    """A non-OK status from libtwnorm."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_STATUS_NAMES = {TW_OK: "TW_OK", TW_ERR_INVALID_ARG: "TW_ERR_INVALID_ARG",
                 TW_ERR_UNSUPPORTED: "TW_ERR_UNSUPPORTED", TW_ERR_ALIAS: "TW_ERR_ALIAS",
                 TW_ERR_HIP: "TW_ERR_HIP"}

EXPORTED = ("tw_fused_reduce_rmsnorm", "tw_fused_reduce_rmsnorm_allgather", "tw_reduce",
            "tw_rmsnorm", "tw_cu_masked_stream", "tw_cu_complement_stream", "tw_shutdown",
            "tw_status_string", "tw_last_error", "tw_abi_version",
            # measurement and tuning aids (include/twnorm_bench.h)
            "tw_stream_copy", "tw_stream_mix", "tw_set_fused_shape", "tw_query_fused_shape")


def _hip_runtimes_loaded():
    """Distinct HIP runtime files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtwnorm.so (once).  Raises if it has not been built.

    torch is imported first so that the library binds to the HIP runtime
    torch already uses: tensors, streams and kernels must all live in one
    runtime.  Loading the library first would map a second HIP runtime into
    the process, which then fails to find the device; that case is detected
    and reported."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m reduce_residual_add_amd.build` (no CPU fallback exists)")
    import torch  # noqa: F401  (binds the HIP runtime torch ships)
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes_loaded()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded in this process "
                          f"({', '.join(sorted(runtimes))}); import torch before loading "
                          "libtwnorm by any other route")
    lib.tw_fused_reduce_rmsnorm.argtypes = [_c.POINTER(_vp), _c.c_int, _i64, _i64, _c.c_int, _vp,
                                            _vp, _c.c_float, _vp, _vp, _c.c_int, _vp]
    lib.tw_fused_reduce_rmsnorm.restype = _c.c_int
    lib.tw_fused_reduce_rmsnorm_allgather.argtypes = [
        _c.POINTER(_vp), _c.c_int, _i64, _i64, _c.c_int, _vp, _vp, _c.c_float, _c.POINTER(_vp),
        _c.c_int, _i64, _i64, _vp, _c.c_int, _vp]
    lib.tw_fused_reduce_rmsnorm_allgather.restype = _c.c_int
    lib.tw_reduce.argtypes = [_c.POINTER(_vp), _c.c_int, _i64, _i64, _c.c_int, _vp, _c.c_int, _vp]
    lib.tw_reduce.restype = _c.c_int
    lib.tw_rmsnorm.argtypes = [_vp, _i64, _i64, _c.c_int, _vp, _vp, _c.c_float, _vp, _vp,
                               _c.c_int, _vp]
    lib.tw_rmsnorm.restype = _c.c_int
    lib.tw_stream_copy.argtypes = [_vp, _vp, _i64, _c.c_int, _vp]
    lib.tw_stream_copy.restype = _c.c_int
    lib.tw_stream_mix.argtypes = [_c.POINTER(_vp), _c.c_int, _c.POINTER(_vp), _c.c_int, _i64,
                                  _c.c_int, _vp]
    lib.tw_stream_mix.restype = _c.c_int
    lib.tw_cu_masked_stream.argtypes = [_c.c_int, _c.POINTER(_vp)]
    lib.tw_cu_masked_stream.restype = _c.c_int
    lib.tw_cu_complement_stream.argtypes = [_c.c_int, _c.POINTER(_vp)]
    lib.tw_cu_complement_stream.restype = _c.c_int
    lib.tw_set_fused_shape.argtypes = [_c.c_int, _c.c_int, _c.c_int]
    lib.tw_set_fused_shape.restype = _c.c_int
    lib.tw_query_fused_shape.argtypes = [_c.c_int, _i64, _c.c_int, _i64, _c.c_int, _c.c_int,
                                         _c.POINTER(_c.c_int),
                                         _c.POINTER(_c.c_int), _c.POINTER(_c.c_int)]
    lib.tw_query_fused_shape.restype = _c.c_int
    lib.tw_shutdown.argtypes = []
    lib.tw_shutdown.restype = _c.c_int
    lib.tw_status_string.argtypes = [_c.c_int]
    lib.tw_status_string.restype = _c.c_char_p
    lib.tw_last_error.argtypes = []
    lib.tw_last_error.restype = _c.c_char_p
    lib.tw_abi_version.argtypes = []
    lib.tw_abi_version.restype = _c.c_int
    if lib.tw_abi_version() != TW_ABI_VERSION:
        raise ImportError(f"libtwnorm ABI {lib.tw_abi_version()} != {TW_ABI_VERSION}")
    # Release the CU-masked streams while torch and the HIP runtime are fully
    # alive: Python's exit hooks run before any C-level teardown.
    atexit.register(lib.tw_shutdown)
    _lib = lib
    return lib


def last_error() -> str:
    return load().tw_last_error().decode()


def _check(status: int) -> None:
    if status != TW_OK:
        raise TwError(status, last_error())


# ---------------------------------------------------------------------------
# torch plumbing (device memory, dtype tag, current stream)
# ---------------------------------------------------------------------------


def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TW_BF16
    if t.dtype == torch.float32:
        return TW_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_tensor(t, name: str, shape, dt, device) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dt:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dt}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(stream=None) -> int:
    """The hipStream_t of `stream`, else of the current device's current
    stream (read without building a Stream object when torch offers it)."""
    if stream is not None:
        return int(stream.cuda_stream)
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(torch._C._cuda_getDevice()))
    return int(torch.cuda.current_stream().cuda_stream)


def _stream_device_index(stream):
    """Device index of a torch stream object, or None if it does not say."""
    sdev = getattr(stream, "device", None)
    return None if sdev is None else sdev.index


def _check_device(index: int, stream=None) -> None:
    """The tensors' device `index` and `stream`'s device must be the current
    device: the library launches there and takes its CU count from it."""
    cur = _torch()._C._cuda_getDevice()
    if index != cur:
        raise ValueError(f"the tensors are on cuda:{index} but the current device is cuda:{cur}; "
                         f"call inside torch.cuda.device({index})")
    if stream is not None:
        sidx = _stream_device_index(stream)
        if sidx is not None and sidx != cur:
            raise ValueError(f"the stream is on cuda:{sidx} but the current device is cuda:{cur}")


def _rows_hidden(t):
    if t.dim() != 2:
        raise ValueError("tensors are [rows, hidden]")
    return int(t.shape[0]), int(t.shape[1])


def _check_fused_tensors(partials, residual, weight, out, residual_out, stream=None):
    """Device, dtype, shape and contiguity of a fused call's tensors; returns
    (rows, hidden, n).  One combined test per tensor on the common path; the
    per-property checks below run only to word the error."""
    shape = residual.shape
    n = len(partials)
    if len(shape) == 2 and residual.is_cuda and 1 <= n <= TW_MAX_PARTIALS:
        dt, dev = residual.dtype, residual.get_device()
        wshape = shape[1:]
        ok = (dev == _torch()._C._cuda_getDevice() and
              (stream is None or _stream_device_index(stream) in (None, dev)) and
              residual.is_contiguous() and
              weight.is_cuda and weight.dtype is dt and weight.get_device() == dev and
              weight.shape == wshape and weight.is_contiguous())
        if ok:
            for t in (out, residual_out, *partials):
                if not (t.is_cuda and t.dtype is dt and t.get_device() == dev and t.shape == shape
                        and t.is_contiguous()):
                    ok = False
                    break
        if ok:
            return int(shape[0]), int(shape[1]), n
    return _check_fused_tensors_slow(partials, residual, weight, out, residual_out, stream)


def _check_fused_tensors_slow(partials, residual, weight, out, residual_out, stream=None):
    rows, hidden = _rows_hidden(residual)
    dt, dev = residual.dtype, residual.device
    n = len(partials)
    if n < 1 or n > TW_MAX_PARTIALS:
        raise ValueError(f"need 1..{TW_MAX_PARTIALS} partials, got {n}")
    for i, p in enumerate(partials):
        _check_tensor(p, f"partials[{i}]", (rows, hidden), dt, dev)
    _check_tensor(residual, "residual", (rows, hidden), dt, dev)
    _check_tensor(weight, "weight", (hidden,), dt, dev)
    _check_tensor(out, "out", (rows, hidden), dt, dev)
    _check_tensor(residual_out, "residual_out", (rows, hidden), dt, dev)
    _check_device(dev.index, stream)
    return rows, hidden, n


_DTYPE_CODES = {}


def _dtype_code_fast(t) -> int:
    c = _DTYPE_CODES.get(t.dtype)
    if c is None:
        c = _DTYPE_CODES[t.dtype] = dtype_code(t)
    return c


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------


def fused_reduce_rmsnorm(partials: Sequence, residual, weight, eps: float, *, out=None,
                         residual_out=None, n_cu_limit: int = 0, stream=None):
    """out = RMSNorm(residual + sum(partials)) * weight; residual_out =
    residual + sum(partials).  Pass ``residual_out=residual`` for the in-place
    residual update.  Returns (out, residual_out)."""
    torch = _torch()
    lib = load()
    if out is None:
        out = torch.empty_like(residual)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    rows, hidden, n = _check_fused_tensors(partials, residual, weight, out, residual_out, stream)
    if rows == 0:   # nothing to do (an empty tensor's data_ptr() may be NULL)
        return out, residual_out
    arr = (_vp * n)(*[p.data_ptr() for p in partials])
    _check(lib.tw_fused_reduce_rmsnorm(arr, n, rows, hidden, _dtype_code_fast(residual),
                                       residual.data_ptr(), weight.data_ptr(), float(eps),
                                       out.data_ptr(), residual_out.data_ptr(), int(n_cu_limit),
                                       _stream_ptr(stream)))
    return out, residual_out


def fused_reduce_rmsnorm_allgather(partials: Sequence, residual, weight, eps: float,
                                   ag_outs: Sequence, ag_row_offset: int, *, residual_out=None,
                                   n_cu_limit: int = 0, stream=None):
    """Fused step with the AllGather store: the normalised rows go to rows
    [ag_row_offset, ag_row_offset + rows) of every buffer in `ag_outs`
    (each [T, hidden]).  Returns residual_out."""
    torch = _torch()
    lib = load()
    rows, hidden = _rows_hidden(residual)
    dt, dev = residual.dtype, residual.device
    n, n_ag = len(partials), len(ag_outs)
    if n < 1 or n > TW_MAX_PARTIALS or n_ag < 1 or n_ag > TW_MAX_PARTIALS:
        raise ValueError(f"need 1..{TW_MAX_PARTIALS} partials and gather buffers")
    for i, p in enumerate(partials):
        _check_tensor(p, f"partials[{i}]", (rows, hidden), dt, dev)
    _check_tensor(residual, "residual", (rows, hidden), dt, dev)
    _check_tensor(weight, "weight", (hidden,), dt, dev)
    total = int(ag_outs[0].shape[0])
    for j, g in enumerate(ag_outs):
        _check_tensor(g, f"ag_outs[{j}]", (total, hidden), dt, dev)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _check_tensor(residual_out, "residual_out", (rows, hidden), dt, dev)
    _check_device(dev.index, stream)
    if rows == 0:
        return residual_out
    arr = (_vp * n)(*[p.data_ptr() for p in partials])
    ag = (_vp * n_ag)(*[g.data_ptr() for g in ag_outs])
    _check(lib.tw_fused_reduce_rmsnorm_allgather(
        arr, n, rows, hidden, dtype_code(residual), residual.data_ptr(), weight.data_ptr(),
        float(eps), ag, n_ag, int(ag_row_offset), total, residual_out.data_ptr(), int(n_cu_limit),
        _stream_ptr(stream)))
    return residual_out


def reduce(partials: Sequence, *, out=None, n_cu_limit: int = 0, stream=None):
    """reduced = sum(partials), rounded to the storage dtype (the unfused
    path's HBM intermediate).  Returns ``reduced``."""
    torch = _torch()
    lib = load()
    n = len(partials)
    if n < 1 or n > TW_MAX_PARTIALS:
        raise ValueError(f"need 1..{TW_MAX_PARTIALS} partials, got {n}")
    rows, hidden = _rows_hidden(partials[0])
    dt, dev = partials[0].dtype, partials[0].device
    for i, p in enumerate(partials):
        _check_tensor(p, f"partials[{i}]", (rows, hidden), dt, dev)
    if out is None:
        out = torch.empty_like(partials[0])
    _check_tensor(out, "out", (rows, hidden), dt, dev)
    _check_device(dev.index, stream)
    if rows == 0:
        return out
    arr = (_vp * n)(*[p.data_ptr() for p in partials])
    _check(lib.tw_reduce(arr, n, rows, hidden, dtype_code(out), out.data_ptr(), int(n_cu_limit),
                         _stream_ptr(stream)))
    return out


def rmsnorm(reduced, residual, weight, eps: float, *, out=None, residual_out=None,
            n_cu_limit: int = 0, stream=None):
    """out = RMSNorm(residual + reduced) * weight; residual_out = residual +
    reduced.  The unfused path's second kernel.  Returns (out, residual_out)."""
    torch = _torch()
    lib = load()
    rows, hidden = _rows_hidden(residual)
    dt, dev = residual.dtype, residual.device
    _check_tensor(reduced, "reduced", (rows, hidden), dt, dev)
    _check_tensor(residual, "residual", (rows, hidden), dt, dev)
    _check_tensor(weight, "weight", (hidden,), dt, dev)
    if out is None:
        out = torch.empty_like(residual)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    _check_tensor(out, "out", (rows, hidden), dt, dev)
    _check_tensor(residual_out, "residual_out", (rows, hidden), dt, dev)
    _check_device(dev.index, stream)
    if rows == 0:
        return out, residual_out
    _check(lib.tw_rmsnorm(reduced.data_ptr(), rows, hidden, dtype_code(residual),
                          residual.data_ptr(), weight.data_ptr(), float(eps), out.data_ptr(),
                          residual_out.data_ptr(), int(n_cu_limit), _stream_ptr(stream)))
    return out, residual_out


def _check_raw(tensors, names, nbytes, device) -> None:
    """GPU-resident, contiguous, on one device, each `nbytes` long."""
    for t, name in zip(tensors, names):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() * t.element_size() != nbytes:
            raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, expected {nbytes}")


def stream_copy(src, dst, *, n_cu_limit: int = 0, stream=None):
    """dst = src byte for byte (measurement aid: the plain-copy ceiling)."""
    lib = load()
    nbytes = src.numel() * src.element_size()
    _check_raw((src, dst), ("src", "dst"), nbytes, src.device)
    _check_device(src.device.index, stream)
    _check(lib.tw_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, int(n_cu_limit),
                              _stream_ptr(stream)))
    return dst


def stream_mix(srcs: Sequence, dsts: Sequence, *, n_cu_limit: int = 0, stream=None):
    """Measurement aid: the fused kernel's traffic pattern without its
    arithmetic.  Every 32-bit word of every dst becomes the wrap-around
    uint32 sum of that word over the srcs (all of one byte size)."""
    lib = load()
    n_src, n_dst = len(srcs), len(dsts)
    if n_src < 1 or n_src > TW_MAX_PARTIALS + 1 or n_dst < 1 or n_dst > TW_MAX_PARTIALS:
        raise ValueError(f"need 1..{TW_MAX_PARTIALS + 1} srcs and 1..{TW_MAX_PARTIALS} dsts")
    nbytes = srcs[0].numel() * srcs[0].element_size()
    _check_raw(list(srcs) + list(dsts), [f"srcs[{i}]" for i in range(n_src)] +
               [f"dsts[{j}]" for j in range(n_dst)], nbytes, srcs[0].device)
    _check_device(srcs[0].device.index, stream)
    if nbytes == 0:
        return dsts
    sa = (_vp * n_src)(*[t.data_ptr() for t in srcs])
    da = (_vp * n_dst)(*[t.data_ptr() for t in dsts])
    _check(lib.tw_stream_mix(sa, n_src, da, n_dst, nbytes, int(n_cu_limit), _stream_ptr(stream)))
    return dsts


def cu_masked_stream(n_cu_limit: int):
    """The library's CU-masked stream for `n_cu_limit` CUs, as a torch
    ExternalStream.  Calls issued on it with the same n_cu_limit skip the
    per-call event join (order it against other streams yourself)."""
    torch = _torch()
    h = _vp()
    _check(load().tw_cu_masked_stream(int(n_cu_limit), ctypes.byref(h)))
    return torch.cuda.ExternalStream(h.value)


def cu_complement_stream(n_cu_limit: int):
    """The library's stream on the CUs that `cu_masked_stream(n_cu_limit)`
    leaves free (for other work beside CU-limited fused calls), as a torch
    ExternalStream."""
    torch = _torch()
    h = _vp()
    _check(load().tw_cu_complement_stream(int(n_cu_limit), ctypes.byref(h)))
    return torch.cuda.ExternalStream(h.value)


def shutdown() -> None:
    """Release the library's CU-masked streams and events now (it also runs
    at interpreter exit).  Afterwards CU-limited calls raise; whole-chip
    calls keep working."""
    _check(load().tw_shutdown())


def set_fused_shape(waves: int = 0, chunks_per_lane: int = 0, wgs_per_cu: int = 0) -> None:
    """Force the fused kernel's launch shape (0, 0 = automatic) and, with
    wgs_per_cu > 0, run it on a persistent grid of at most wgs_per_cu
    workgroups per CU (0 = the default grid), for the calling thread's later
    calls."""
    _check(load().tw_set_fused_shape(int(waves), int(chunks_per_lane), int(wgs_per_cu)))


def query_fused_shape(dtype: int, hidden: int, n: int, rows: int = 1 << 40, cus: int = 256,
                      device_cus: int = 256):
    """(waves, chunks_per_lane, team_lanes) the fused kernel uses for n
    partials of rows `hidden` wide when `rows` rows run on `cus` of the
    device's `device_cus` CUs (the defaults: a call large enough to fill a
    whole 256-CU chip)."""
    w, k, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(load().tw_query_fused_shape(int(dtype), int(hidden), int(n), int(rows), int(cus),
                                       int(device_cus), ctypes.byref(w), ctypes.byref(k),
                                       ctypes.byref(t)))
    return w.value, k.value, t.value


class PreparedFused:
    """Pre-marshalled arguments of one fused call, for tight timing loops:
    ``__call__`` is one ctypes call with no per-call conversions."""

    def __init__(self, partials, residual, weight, eps, out, residual_out, n_cu_limit=0,
                 stream=None):
        self._lib = load()
        rows, hidden, self._n = _check_fused_tensors(partials, residual, weight, out, residual_out,
                                                     stream)
        self._rows = rows
        self._keep = (list(partials), residual, weight, out, residual_out)
        self._arr = (_vp * self._n)(*[p.data_ptr() for p in partials])
        self._args = (self._arr, self._n, rows, hidden, dtype_code(residual), residual.data_ptr(),
                      weight.data_ptr(), ctypes.c_float(float(eps)), out.data_ptr(),
                      residual_out.data_ptr(), int(n_cu_limit), _stream_ptr(stream))

    def __call__(self) -> None:
        if self._rows == 0:
            return
        st = self._lib.tw_fused_reduce_rmsnorm(*self._args)
        if st != TW_OK:
            _check(st)
