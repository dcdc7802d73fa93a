"""Python binding of ``libqknorm.so`` (argument marshalling only).

Every function has the C entry point's name without the ``qknorm_`` prefix
and the dtype suffix; the dtype comes from the tensors. PyTorch supplies
device memory and the stream (the current stream of the tensors' device);
all computation runs in the library's HIP kernels. If the library is not
built, the first call raises ``RuntimeError`` -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqknorm.so")
_lib = None
_lock = threading.Lock()

QKN_OK, QKN_EINVAL, QKN_EOVERLAP, QKN_ENOMEM, QKN_EHIP = 0, -1, -2, -3, -4
QKN_ERESIDENCY, QKN_ETIMEOUT, QKN_ECAPTURE, QKN_ESCRATCH = -5, -6, -7, -8
QKN_BF16, QKN_F32, QKN_E4M3 = 0, 1, 2
# kernel formats (input x / gamma / output y), the ``dtype`` of the planning calls
FORMATS = {"bf16": 0, "f32": 1, "e4m3_bf16": 2, "e4m3_e4m3": 3, "ln_bf16": 4, "ln_f32": 5}
E4M3 = torch.float8_e4m3fn
NUM_VARIANTS = 11
MAX_DATA_WAVES = 15
MAX_SHARDS = 64
OPT = {"spin_limit_ns": 1, "force_variant": 2, "rows": 3, "xcd_map": 4, "cooperative": 5,
       "max_groups": 6, "force_split": 7, "test_skip_publish": 8, "data_waves": 9,
       "split_vectors": 10, "tile_layout": 11, "wpc": 12, "static_slots": 13, "pace": 14}


class QKNormError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {strerror(status)} ({status})"
        hip = last_hip_error()
        if hip:
            msg += f" [{hip}]"
        super().__init__(msg)


class Plan(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("threads", ctypes.c_int),
                ("data_waves", ctypes.c_int), ("slots", ctypes.c_int),
                ("rows", ctypes.c_int), ("n_tiles", ctypes.c_int64), ("n_groups", ctypes.c_int),
                ("grid", ctypes.c_int), ("xcd_map", ctypes.c_int), ("iters", ctypes.c_int),
                ("st", ctypes.c_int), ("pace_gbs", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_P, _I64, _I, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
_SIGS = {
    "qknorm_layerwise_fwd_bf16": [_P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _P],
    "qknorm_layerwise_fwd_f32": [_P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _P],
    "qknorm_layerwise_fwd_bf16_noalloc": [_P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _P],
    "qknorm_layerwise_fwd_e4m3": [_P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _I, _P],
    "qknorm_shard_sumsq_bf16": [_P, _I64, _I64, _I, _P, _P],
    "qknorm_shard_sumsq_f32": [_P, _I64, _I64, _I, _P, _P],
    "qknorm_shard_sumsq_e4m3": [_P, _I64, _I64, _I, _P, _P],
    "qknorm_combine_scale": [_P, _I64, _I64, _I, _F, _P, _P],
    "qknorm_apply_scale_bf16": [_P, _P, _P, _I64, _I64, _P, _P],
    "qknorm_apply_scale_f32": [_P, _P, _P, _I64, _I64, _P, _P],
    "qknorm_apply_scale_e4m3": [_P, _P, _P, _I64, _I64, _P, _I, _P],
    "qknorm_layernorm_fwd_bf16": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _P],
    "qknorm_layernorm_fwd_f32": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _P],
    "qknorm_shard_stats_bf16": [_P, _I64, _I64, _I, _P, _P, _P],
    "qknorm_shard_stats_f32": [_P, _I64, _I64, _I, _P, _P, _P],
    "qknorm_combine_stats": [_P, _P, _I64, _I64, _I, _F, _P, _P, _P],
    "qknorm_apply_norm_bf16": [_P, _P, _P, _P, _P, _I64, _I64, _P, _P],
    "qknorm_apply_norm_f32": [_P, _P, _P, _P, _P, _I64, _I64, _P, _P],
    "qknorm_headwise_fwd_bf16": [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _P, _P, _P],
    "qknorm_headwise_fwd_f32": [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _P, _P, _P],
    "qknorm_check_fault": [_P],
    "qknorm_fault_pending": [],
    "qknorm_fault_flag": [],
    "qknorm_strerror": [_I],
    "qknorm_last_hip_error": [],
    "qknorm_max_coresident_workgroups": [_I, _I64, _I64, _I, ctypes.POINTER(_I)],
    "qknorm_release_workspace": [],
    "qknorm_device_occupancy": [_I, ctypes.POINTER(_I), ctypes.POINTER(_I)],
    "qknorm_plan_fused": [_I, _I64, _I64, _I64, _I, _I, ctypes.POINTER(_I), _I,
                          ctypes.POINTER(Plan)],
    "qknorm_set_option": [_I, _I64],
    "qknorm_get_option": [_I],
    "qknorm_bench_copy": [_P, _P, _P, _P, _I64, _I64, _P],
    "qknorm_bench_widen": [_P, _P, _P, _P, _I64, _I64, _P],
    "qknorm_bench_skeleton": [_I, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P],
    "qknorm_bench_fused": [_I, _P, _P, _P, _P, _I64, _I64, _I64, _I, _F, _P, _P, _I, _P],
}
_RESTYPE = {"qknorm_strerror": ctypes.c_char_p, "qknorm_last_hip_error": ctypes.c_char_p,
            "qknorm_get_option": ctypes.c_int64, "qknorm_fault_flag": ctypes.c_void_p}


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH):
                    raise RuntimeError(
                        f"{_LIB_PATH} is missing: build it with "
                        "`python -m layerwise_qk_norm_amd.build` (there is no fallback path)")
                L = ctypes.CDLL(_LIB_PATH)
                for name, args in _SIGS.items():
                    fn = getattr(L, name)
                    fn.argtypes = args
                    fn.restype = _RESTYPE.get(name, ctypes.c_int)
                _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().qknorm_strerror(status).decode()


def last_hip_error() -> str:
    return lib().qknorm_last_hip_error().decode()


def _check(status: int, what: str):
    if status != QKN_OK:
        raise QKNormError(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return QKN_BF16
    if t.dtype == torch.float32:
        return QKN_F32
    if t.dtype == E4M3:
        return QKN_E4M3
    raise TypeError(f"tensors must be bfloat16, float32 or float8_e4m3fn, got {t.dtype}")


def _suffix(code: int) -> str:
    return {QKN_BF16: "bf16", QKN_F32: "f32", QKN_E4M3: "e4m3"}[code]


def _out_dtype(x_dtype, out, out_dtype):
    """Output dtype of a call: bf16/fp32 inputs keep their dtype; E4M3 inputs
    give bf16 unless E4M3 is asked for (by ``out`` or ``out_dtype``)."""
    if x_dtype != E4M3:
        want = x_dtype
    elif out is not None:
        want = out.dtype
    else:
        want = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype is not None and out_dtype != want:
        raise TypeError(f"out_dtype {out_dtype} does not match the output {want}")
    if x_dtype == E4M3 and want not in (torch.bfloat16, E4M3):
        raise TypeError(f"E4M3 inputs give bfloat16 or float8_e4m3fn outputs, not {want}")
    return want


def _gamma_dtype(x_dtype):
    return torch.bfloat16 if x_dtype == E4M3 else x_dtype


def format_of(x_dtype, out_dtype) -> int:
    """Kernel format code of an input/output dtype pair."""
    if x_dtype == torch.bfloat16:
        return FORMATS["bf16"]
    if x_dtype == torch.float32:
        return FORMATS["f32"]
    return FORMATS["e4m3_bf16" if out_dtype == torch.bfloat16 else "e4m3_e4m3"]


def _need(t: torch.Tensor, name: str, ndim: int, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# The current stream's handle as an int, without building a torch Stream object
# (about a microsecond per call less); the public API when this build lacks it.
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_GET_DEVICE = getattr(torch._C, "_cuda_getDevice", None)


def _raw_stream(index: int) -> int:
    return _RAW_STREAM(index) if _RAW_STREAM is not None else torch.cuda.current_stream(index).cuda_stream


def _current_device() -> int:
    return _GET_DEVICE() if _GET_DEVICE is not None else torch.cuda.current_device()


_FLAGS = {}  # device index -> the device's timeout flag (pinned host word), or None


def _timeout_flag(index: int):
    f = _FLAGS.get(index, False)
    if f is False:
        with torch.cuda.device(index):
            addr = lib().qknorm_fault_flag()
        f = ctypes.c_uint32.from_address(addr) if addr else None
        _FLAGS[index] = f
    return f


def _issue(fn, args, index: int, what: str):
    """Calls a C entry point on the current stream of device ``index``, with that
    device current (the library plans and keeps its workspace per current device).

    Before issuing it reads the device's timeout flag, a word of pinned host memory
    that a fused launch sets when it abandons an exchange: if an earlier call timed
    out, its outputs are unspecified and this raises QKNormError (QKN_ETIMEOUT)
    without issuing, until check_fault() clears the flag."""
    f = _timeout_flag(index)
    if f is not None and f.value:
        raise QKNormError(QKN_ETIMEOUT, f"{what}: an earlier fused call on cuda:{index} timed out "
                          "(its outputs are unspecified; check_fault() clears this)")
    if _current_device() == index:
        status = fn(*args, _raw_stream(index))
    else:
        with torch.cuda.device(index):
            status = fn(*args, _raw_stream(index))
    if status != QKN_OK:
        raise QKNormError(status, what)


class Prepared:
    """A validated call, issued again by calling the object: ``outs = prepared()``.

    Validation (dtypes, shapes, contiguity, devices) runs once, when the object is
    made; each call then only passes the stored pointers and the current stream to
    the library, which still validates sizes, overlap and residency. Meant for
    loops that reuse the same tensors (decode steps, graph-free serving loops).
    The contents of the tensors may change between calls; their shapes and
    storage must not (no ``resize_``, ``set_`` or reallocation), and the object
    keeps them alive. Returns the output tensors.
    """

    __slots__ = ("_fn", "_args", "_index", "_what", "_outs", "_keep")

    def __init__(self, fn, args, index, what, outs, keep):
        self._fn, self._args, self._index, self._what = fn, args, index, what
        self._outs, self._keep = outs, keep

    def __call__(self):
        _issue(self._fn, self._args, self._index, self._what)
        return self._outs


def _layerwise_call(q, k, gamma_q, gamma_k, n_shards, eps, out_q, out_k, out_dtype):
    _need(q, "q", 2)
    dt = q.dtype
    dev = q.device
    code = _dtype_code(q)
    _need(k, "k", 2, dt, dev)
    _need(gamma_q, "gamma_q", 1, _gamma_dtype(dt), dev)
    _need(gamma_k, "gamma_k", 1, _gamma_dtype(dt), dev)
    T, Hq = q.shape
    if k.shape[0] != T:
        raise ValueError("q and k must have the same number of tokens")
    Hk = k.shape[1]
    if gamma_q.shape[0] != Hq or gamma_k.shape[0] != Hk:
        raise ValueError("gamma_q must be [Hq] and gamma_k [Hk]")
    odt = _out_dtype(dt, out_q if out_q is not None else out_k, out_dtype)
    out_q = torch.empty(q.shape, dtype=odt, device=dev) if out_q is None else out_q
    out_k = torch.empty(k.shape, dtype=odt, device=dev) if out_k is None else out_k
    _need(out_q, "out_q", 2, odt, dev)
    _need(out_k, "out_k", 2, odt, dev)
    if out_q.shape != q.shape or out_k.shape != k.shape:
        raise ValueError("outputs must have the shapes of q and k")
    L = lib()
    args = (q.data_ptr(), k.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(), T, Hq, Hk,
            n_shards, eps, out_q.data_ptr(), out_k.data_ptr())
    if code == QKN_E4M3:
        fn = L.qknorm_layerwise_fwd_e4m3
        args = args + (_dtype_code(out_q),)
    else:
        fn = L.qknorm_layerwise_fwd_bf16 if code == QKN_BF16 else L.qknorm_layerwise_fwd_f32
    return Prepared(fn, args, dev.index, "qknorm_layerwise_fwd", (out_q, out_k),
                    (q, k, gamma_q, gamma_k))


def layerwise_fwd(q, k, gamma_q, gamma_k, n_shards: int, eps: float = 1e-6, out_q=None,
                  out_k=None, out_dtype=None):
    """Fused Q+K layerwise RMSNorm; returns ``(out_q, out_k)``.

    q and k are bfloat16, float32 or float8_e4m3fn (E4M3). gamma has the dtype of
    q, except bfloat16 for E4M3 inputs. Outputs have the dtype of q, except for
    E4M3 inputs: bfloat16 by default, float8_e4m3fn when ``out_dtype`` (or the
    given outputs) say so.
    """
    return _layerwise_call(q, k, gamma_q, gamma_k, n_shards, eps, out_q, out_k, out_dtype)()


def prepare_layerwise_fwd(q, k, gamma_q, gamma_k, n_shards: int, eps: float = 1e-6, out_q=None,
                          out_k=None, out_dtype=None) -> Prepared:
    """``layerwise_fwd`` validated once: the returned object issues the call each
    time it is called (see ``Prepared``)."""
    return _layerwise_call(q, k, gamma_q, gamma_k, n_shards, eps, out_q, out_k, out_dtype)


def _ptr_or_null(t):
    return None if t is None else t.data_ptr()


def _layernorm_call(q, k, gamma_q, gamma_k, n_shards, eps, beta_q, beta_k, out_q, out_k):
    _need(q, "q", 2)
    dt = q.dtype
    dev = q.device
    code = _dtype_code(q)
    if code == QKN_E4M3:
        raise TypeError("LayerNorm takes bfloat16 or float32 tensors")
    _need(k, "k", 2, dt, dev)
    T, Hq = q.shape
    Hk = k.shape[1]
    if k.shape[0] != T:
        raise ValueError("q and k must have the same number of tokens")
    for t, name, H in ((gamma_q, "gamma_q", Hq), (gamma_k, "gamma_k", Hk),
                       (beta_q, "beta_q", Hq), (beta_k, "beta_k", Hk)):
        if t is None and name.startswith("beta"):
            continue
        _need(t, name, 1, dt, dev)
        if t.shape[0] != H:
            raise ValueError(f"{name} must be [{H}]")
    out_q = torch.empty_like(q) if out_q is None else out_q
    out_k = torch.empty_like(k) if out_k is None else out_k
    _need(out_q, "out_q", 2, dt, dev)
    _need(out_k, "out_k", 2, dt, dev)
    if out_q.shape != q.shape or out_k.shape != k.shape:
        raise ValueError("outputs must have the shapes of q and k")
    fn = getattr(lib(), f"qknorm_layernorm_fwd_{_suffix(code)}")
    args = (q.data_ptr(), k.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(),
            _ptr_or_null(beta_q), _ptr_or_null(beta_k), T, Hq, Hk, n_shards, eps,
            out_q.data_ptr(), out_k.data_ptr())
    return Prepared(fn, args, dev.index, "qknorm_layernorm_fwd", (out_q, out_k),
                    (q, k, gamma_q, gamma_k, beta_q, beta_k))


def layernorm_fwd(q, k, gamma_q, gamma_k, n_shards: int, eps: float = 1e-5, beta_q=None,
                  beta_k=None, out_q=None, out_k=None):
    """Fused Q+K LayerNorm over the full vectors with two additive shard statistics;
    returns ``(out_q, out_k)``. bfloat16 or float32; beta may be None (no shift)."""
    return _layernorm_call(q, k, gamma_q, gamma_k, n_shards, eps, beta_q, beta_k, out_q, out_k)()


def prepare_layernorm_fwd(q, k, gamma_q, gamma_k, n_shards: int, eps: float = 1e-5, beta_q=None,
                          beta_k=None, out_q=None, out_k=None) -> Prepared:
    """``layernorm_fwd`` validated once (see ``Prepared``)."""
    return _layernorm_call(q, k, gamma_q, gamma_k, n_shards, eps, beta_q, beta_k, out_q, out_k)


def _headwise_call(q, k, gamma_q, gamma_k, head_dim, eps, out_q, out_k):
    _need(q, "q", 2)
    dt = q.dtype
    dev = q.device
    code = _dtype_code(q)
    if code == QKN_E4M3:
        raise TypeError("headwise takes bfloat16 or float32 tensors")
    _need(k, "k", 2, dt, dev)
    _need(gamma_q, "gamma_q", 1, dt, dev)
    _need(gamma_k, "gamma_k", 1, dt, dev)
    T, Hq = q.shape
    Hk = k.shape[1]
    if k.shape[0] != T:
        raise ValueError("q and k must have the same number of tokens")
    if head_dim < 1 or Hq % head_dim or Hk % head_dim:
        raise ValueError("q and k rows must be whole heads of head_dim columns")
    if gamma_q.shape[0] != head_dim or gamma_k.shape[0] != head_dim:
        raise ValueError("gamma_q and gamma_k must be [head_dim]")
    out_q = torch.empty_like(q) if out_q is None else out_q
    out_k = torch.empty_like(k) if out_k is None else out_k
    _need(out_q, "out_q", 2, dt, dev)
    _need(out_k, "out_k", 2, dt, dev)
    if out_q.shape != q.shape or out_k.shape != k.shape:
        raise ValueError("outputs must have the shapes of q and k")
    fn = getattr(lib(), f"qknorm_headwise_fwd_{_suffix(code)}")
    args = (q.data_ptr(), k.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(), T,
            Hq // head_dim, Hk // head_dim, head_dim, eps, out_q.data_ptr(), out_k.data_ptr())
    return Prepared(fn, args, dev.index, "qknorm_headwise_fwd", (out_q, out_k),
                    (q, k, gamma_q, gamma_k))


def headwise_fwd(q, k, gamma_q, gamma_k, head_dim: int, eps: float = 1e-6, out_q=None,
                 out_k=None):
    """Headwise RMSNorm of q and k (one factor per head of ``head_dim`` columns;
    gamma_q and gamma_k are [head_dim]); returns ``(out_q, out_k)``."""
    return _headwise_call(q, k, gamma_q, gamma_k, head_dim, eps, out_q, out_k)()


def prepare_headwise_fwd(q, k, gamma_q, gamma_k, head_dim: int, eps: float = 1e-6, out_q=None,
                         out_k=None) -> Prepared:
    """``headwise_fwd`` validated once (see ``Prepared``)."""
    return _headwise_call(q, k, gamma_q, gamma_k, head_dim, eps, out_q, out_k)


def shard_stats(x, n_shards: int, sums=None, sumsq=None):
    """Per-shard fp32 sums and sums of squares, each ``[n_shards, T]``."""
    _need(x, "x", 2)
    T, H = x.shape
    code = _dtype_code(x)
    if code == QKN_E4M3:
        raise TypeError("LayerNorm takes bfloat16 or float32 tensors")
    sums = torch.empty((n_shards, T), dtype=torch.float32, device=x.device) if sums is None else sums
    sumsq = torch.empty((n_shards, T), dtype=torch.float32, device=x.device) if sumsq is None else sumsq
    for t, name in ((sums, "sums"), (sumsq, "sumsq")):
        _need(t, name, 2, torch.float32, x.device)
        if tuple(t.shape) != (n_shards, T):
            raise ValueError(f"{name} must be [n_shards, T]")
    fn = getattr(lib(), f"qknorm_shard_stats_{_suffix(code)}")
    with torch.cuda.device(x.device):
        _check(fn(x.data_ptr(), T, H, n_shards, sums.data_ptr(), sumsq.data_ptr(),
                  _stream(x.device)), "qknorm_shard_stats")
    return sums, sumsq


def combine_stats(sums, sumsq, H: int, eps: float = 1e-5, mean=None, rstd=None):
    """Mean and reciprocal standard deviation per token, each ``[T]`` fp32."""
    _need(sums, "sums", 2, torch.float32)
    _need(sumsq, "sumsq", 2, torch.float32, sums.device)
    n_shards, T = sums.shape
    if tuple(sumsq.shape) != (n_shards, T):
        raise ValueError("sums and sumsq must have the same shape")
    mean = torch.empty((T,), dtype=torch.float32, device=sums.device) if mean is None else mean
    rstd = torch.empty((T,), dtype=torch.float32, device=sums.device) if rstd is None else rstd
    _need(mean, "mean", 1, torch.float32, sums.device)
    _need(rstd, "rstd", 1, torch.float32, sums.device)
    with torch.cuda.device(sums.device):
        _check(lib().qknorm_combine_stats(sums.data_ptr(), sumsq.data_ptr(), T, H, n_shards, eps,
                                          mean.data_ptr(), rstd.data_ptr(), _stream(sums.device)),
               "qknorm_combine_stats")
    return mean, rstd


def apply_norm(x, gamma, beta, mean, rstd, out=None):
    """``out = (x*gamma)*rstd + (beta - mean*rstd*gamma)`` in x's dtype (beta may be None)."""
    _need(x, "x", 2)
    T, H = x.shape
    code = _dtype_code(x)
    if code == QKN_E4M3:
        raise TypeError("LayerNorm takes bfloat16 or float32 tensors")
    _need(gamma, "gamma", 1, x.dtype, x.device)
    if beta is not None:
        _need(beta, "beta", 1, x.dtype, x.device)
    _need(mean, "mean", 1, torch.float32, x.device)
    _need(rstd, "rstd", 1, torch.float32, x.device)
    out = torch.empty_like(x) if out is None else out
    _need(out, "out", 2, x.dtype, x.device)
    fn = getattr(lib(), f"qknorm_apply_norm_{_suffix(code)}")
    with torch.cuda.device(x.device):
        _check(fn(x.data_ptr(), gamma.data_ptr(), _ptr_or_null(beta), mean.data_ptr(),
                  rstd.data_ptr(), T, H, out.data_ptr(), _stream(x.device)), "qknorm_apply_norm")
    return out


def shard_sumsq(x, n_shards: int, partials=None):
    """Per-shard fp32 sums of squares, ``[n_shards, T]`` (shard-major)."""
    _need(x, "x", 2)
    T, H = x.shape
    if partials is None:
        partials = torch.empty((n_shards, T), dtype=torch.float32, device=x.device)
    _need(partials, "partials", 2, torch.float32, x.device)
    if tuple(partials.shape) != (n_shards, T):
        raise ValueError("partials must be [n_shards, T]")
    code = _dtype_code(x)
    fn = getattr(lib(), f"qknorm_shard_sumsq_{_suffix(code)}")
    with torch.cuda.device(x.device):
        _check(fn(x.data_ptr(), T, H, n_shards, partials.data_ptr(), _stream(x.device)),
               "qknorm_shard_sumsq")
    return partials


def combine_scale(partials, H: int, eps: float = 1e-6, rms_inv=None):
    """Reciprocal RMS per token from shard partials; ``[T]`` fp32."""
    _need(partials, "partials", 2, torch.float32)
    n_shards, T = partials.shape
    if rms_inv is None:
        rms_inv = torch.empty((T,), dtype=torch.float32, device=partials.device)
    _need(rms_inv, "rms_inv", 1, torch.float32, partials.device)
    if rms_inv.shape[0] != T:
        raise ValueError("rms_inv must be [T]")
    with torch.cuda.device(partials.device):
        _check(lib().qknorm_combine_scale(partials.data_ptr(), T, H, n_shards, eps,
                                          rms_inv.data_ptr(), _stream(partials.device)),
               "qknorm_combine_scale")
    return rms_inv


def apply_scale(x, gamma, rms_inv, out=None, out_dtype=None):
    """``out = x * gamma * rms_inv[:, None]`` rounded to the output dtype (x's dtype;
    for E4M3 x: bfloat16 or float8_e4m3fn, with bfloat16 gamma)."""
    _need(x, "x", 2)
    T, H = x.shape
    code = _dtype_code(x)
    _need(gamma, "gamma", 1, _gamma_dtype(x.dtype), x.device)
    _need(rms_inv, "rms_inv", 1, torch.float32, x.device)
    if gamma.shape[0] != H or rms_inv.shape[0] != T:
        raise ValueError("gamma must be [H] and rms_inv [T]")
    odt = _out_dtype(x.dtype, out, out_dtype)
    out = torch.empty(x.shape, dtype=odt, device=x.device) if out is None else out
    _need(out, "out", 2, odt, x.device)
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    fn = getattr(lib(), f"qknorm_apply_scale_{_suffix(code)}")
    args = (x.data_ptr(), gamma.data_ptr(), rms_inv.data_ptr(), T, H, out.data_ptr())
    if code == QKN_E4M3:
        args = args + (_dtype_code(out),)
    with torch.cuda.device(x.device):
        _check(fn(*args, _stream(x.device)), "qknorm_apply_scale")
    return out


def fault_pending(device=None) -> bool:
    """Whether a fused launch on the device has timed out since the last
    check_fault(), without synchronising (launches still running are not seen)."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    with torch.cuda.device(device):
        return bool(lib().qknorm_fault_pending())


def check_fault(device=None) -> int:
    """Synchronise the current stream and return (and clear) its fault status, the
    static scratch arrays' and the device's timeout flag."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    with torch.cuda.device(device):
        return lib().qknorm_check_fault(_stream(device))


def set_option(name: str, value: int):
    _check(lib().qknorm_set_option(OPT[name], int(value)), f"qknorm_set_option({name})")


def get_option(name: str) -> int:
    return int(lib().qknorm_get_option(OPT[name]))


def plan_fused(dtype: str, T: int, Hq: int, Hk: int, n_shards: int, cu_count: int,
               blocks_per_cu, aligned: bool = True) -> dict:
    """Host-only launch plan for a device with the given capacity (no GPU needed).

    ``dtype`` names a format of ``FORMATS``. ``blocks_per_cu[v][w]``: co-resident
    workgroups per CU of variant v with w data waves (NUM_VARIANTS x
    (MAX_DATA_WAVES + 1)).
    """
    flat = [int(x) for row in blocks_per_cu for x in row]
    assert len(flat) == NUM_VARIANTS * (MAX_DATA_WAVES + 1)
    arr = (ctypes.c_int * len(flat))(*flat)
    pl = Plan()
    _check(lib().qknorm_plan_fused(FORMATS[dtype], T, Hq, Hk, n_shards, cu_count, arr,
                                   1 if aligned else 0, ctypes.byref(pl)),
           "qknorm_plan_fused")
    return pl.as_dict()


def max_coresident_workgroups(dtype: str, Hq: int, Hk: int, n_shards: int) -> int:
    out = ctypes.c_int(0)
    _check(lib().qknorm_max_coresident_workgroups(FORMATS[dtype], Hq, Hk, n_shards,
                                                  ctypes.byref(out)),
           "qknorm_max_coresident_workgroups")
    return out.value


def device_occupancy(dtype: str):
    """(blocks_per_cu[variant][data_waves], compute units) of the current device for
    the format ``dtype`` (a key of ``FORMATS``)."""
    arr = (ctypes.c_int * (NUM_VARIANTS * (MAX_DATA_WAVES + 1)))()
    cu = ctypes.c_int(0)
    _check(lib().qknorm_device_occupancy(FORMATS[dtype], arr, ctypes.byref(cu)),
           "qknorm_device_occupancy")
    w = MAX_DATA_WAVES + 1
    return [list(arr[v * w:(v + 1) * w]) for v in range(NUM_VARIANTS)], cu.value


def current_plan(dtype: str, T: int, Hq: int, Hk: int, n_shards: int, aligned: bool = True):
    """The plan the library uses for this shape on the current device."""
    bpc, cu = device_occupancy(dtype)
    return plan_fused(dtype, T, Hq, Hk, n_shards, cu, bpc, aligned)


def bench_copy(q, k, out_q, out_k):
    with torch.cuda.device(q.device):
        _check(lib().qknorm_bench_copy(q.data_ptr(), k.data_ptr(), out_q.data_ptr(),
                                       out_k.data_ptr(), q.numel() * q.element_size(),
                                       k.numel() * k.element_size(), _stream(q.device)),
               "qknorm_bench_copy")


def bench_widen(q, k, out_q, out_k):
    """Ceiling for 1-byte inputs with 2-byte outputs: out = the input bytes zero-extended
    to 16-bit words (``out_q`` and ``out_k`` hold twice the bytes of ``q`` and ``k``)."""
    nq, nk = q.numel() * q.element_size(), k.numel() * k.element_size()
    if out_q.numel() * out_q.element_size() != 2 * nq or out_k.numel() * out_k.element_size() != 2 * nk:
        raise ValueError("outputs must hold twice the bytes of the inputs")
    with torch.cuda.device(q.device):
        _check(lib().qknorm_bench_widen(q.data_ptr(), k.data_ptr(), out_q.data_ptr(),
                                        out_k.data_ptr(), nq, nk, _stream(q.device)),
               "qknorm_bench_widen")


def bench_skeleton(q, k, out_q, out_k, n_shards: int, fmt: str = ""):
    """The fused call's launch plan for this shape run as a copy (no arithmetic, no
    exchange): out = the input bytes, or each byte zero-extended when the output
    element is twice the input's. ``fmt`` names a format of ``FORMATS`` (by default
    the RMSNorm format of the tensors' dtypes)."""
    T, Hq = q.shape
    Hk = k.shape[1]
    f = FORMATS[fmt] if fmt else format_of(q.dtype, out_q.dtype)
    with torch.cuda.device(q.device):
        _check(lib().qknorm_bench_skeleton(f, q.data_ptr(), k.data_ptr(), out_q.data_ptr(), out_k.data_ptr(),
                                           T, Hq, Hk, n_shards, _stream(q.device)), "qknorm_bench_skeleton")


def bench_fused(q, k, gamma_q, gamma_k, n_shards: int, eps: float, out_q, out_k, repeats: int):
    """Issue ``repeats`` back-to-back fused calls from C (measurement helper)."""
    T, Hq = q.shape
    Hk = k.shape[1]
    with torch.cuda.device(q.device):
        _check(lib().qknorm_bench_fused(format_of(q.dtype, out_q.dtype), q.data_ptr(), k.data_ptr(),
                                        gamma_q.data_ptr(), gamma_k.data_ptr(), T, Hq, Hk,
                                        n_shards, eps, out_q.data_ptr(), out_k.data_ptr(),
                                        repeats, _stream(q.device)), "qknorm_bench_fused")


def release_workspace():
    _check(lib().qknorm_release_workspace(), "qknorm_release_workspace")
