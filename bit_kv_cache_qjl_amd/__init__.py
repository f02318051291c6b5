"""Python binding of libqjl (1-bit QJL KV-cache keys on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of libqjl.so, reached
through its C ABI (include/qjl.h).  PyTorch supplies device memory and the current stream.  The
library must be built first (python bit_kv_cache_qjl_amd/build.py); importing this package without
it raises, and there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from . import layout  # noqa: F401  (host-side views of the cache layout)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqjl.so")

QJL_OK = 0
QJL_ERR_INVALID_ARG = -1
QJL_ERR_UNSUPPORTED = -2
QJL_ERR_MISALIGNED = -3
QJL_ERR_WORKSPACE = -4
QJL_ERR_HIP = -5
QJL_BF16 = 0
QJL_F32 = 1
QJL_V_CODES = 0
QJL_V_F32 = 1
QJL_EST_ONE_SIDED = 0
QJL_EST_TWO_SIDED = 1
NO_ALLOC_SCRATCH_BYTES = 8 << 20    # QJL_NO_ALLOC_SCRATCH_BYTES: the fixed workspace of qjl_decode_step_no_alloc

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python bit_kv_cache_qjl_amd/build.py`")

# PyTorch ships its own HIP runtime.  Load it before libqjl so that the library's HIP calls bind to
# the runtime instance that owns the tensors' device memory (loaded the other way round, a process
# can hold two runtimes and the library's launches find no device).
try:
    import torch  # noqa: F401
except ImportError:  # the C ABI alone (argument checks) still works without torch
    torch = None

lib = ctypes.CDLL(LIB_PATH)

_i, _i64, _p, _f, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t

lib.qjl_quantize_keys.restype = _i
lib.qjl_quantize_keys.argtypes = [_p, _i, _i, _i64, _i, _i, _i64, _i64, _i64, _p, _i, _p, _i, _p, _i,
                                  _p, _p, _i64, _i64, _p]
lib.qjl_quantize_values.restype = _i
lib.qjl_quantize_values.argtypes = [_p, _i, _i, _i64, _i, _i, _i64, _i64, _i64, _i, _p, _p, _i64, _i64, _p]
lib.qjl_decode_workspace_size.restype = _sz
lib.qjl_decode_workspace_size.argtypes = [_i, _i, _i, _i, _i64, _i, _i, _i]
lib.qjl_decode_attention.restype = _i
lib.qjl_decode_attention.argtypes = [_p, _i, _i, _i, _i, _i, _i64, _p, _i, _p, _i, _p, _i, _p, _p, _i64,
                                     _i, _p, _p, _p, _i, _f, _i, _p, _p, _i, _p, _sz, _p]
lib.qjl_decode_step.restype = _i
lib.qjl_decode_step.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64, _p, _i, _p, _i, _p, _i,
                                _p, _p, _p, _p, _i64, _i, _f, _i, _p, _p, _i, _p, _sz, _p]
lib.qjl_decode_step_no_alloc.restype = _i
lib.qjl_decode_step_no_alloc.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64, _p, _i, _p, _i, _p,
                                         _i, _p, _p, _p, _p, _i64, _i, _f, _i, _p, _p, _i, _p]
lib.qjl_select_outliers_workspace_size.restype = _sz
lib.qjl_select_outliers_workspace_size.argtypes = [_i, _i64, _i, _i]
lib.qjl_select_outliers.restype = _i
lib.qjl_select_outliers.argtypes = [_p, _i, _i, _i64, _i, _i, _i64, _i64, _i64, _i, _p, _p, _sz, _p]
lib.qjl_status_string.restype = ctypes.c_char_p
lib.qjl_status_string.argtypes = [_i]
lib.qjl_last_error.restype = ctypes.c_char_p
lib.qjl_last_error.argtypes = []
lib.qjl_timer_enable.restype = _i
lib.qjl_timer_enable.argtypes = [_i]
lib.qjl_timer_read.restype = _i
lib.qjl_timer_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double)]


class QJLError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.qjl_status_string(status).decode()} ({status}): "
                         f"{lib.qjl_last_error().decode()}")


def _check(status: int, where: str) -> None:
    if status != QJL_OK:
        raise QJLError(status, where)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _contiguous(**tensors) -> None:
    """The C ABI takes row-major arrays: refuse strided views instead of reading the wrong bytes."""
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor (row-major layout of include/qjl.h)")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return QJL_BF16
    if t.dtype == torch.float32:
        return QJL_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def status_string(status: int) -> str:
    return lib.qjl_status_string(status).decode()


def last_error() -> str:
    return lib.qjl_last_error().decode()


@dataclass
class Cache:
    """Device arrays of one layer's compressed KV cache (layout in include/qjl.h)."""

    bits: object      # int32 view of uint32 [B, Hkv, Ncap, W]
    norms: object     # float16 [B, Hkv, Ncap, 2]
    codes: object     # int32 view of uint32 code tiles [B, Hkv, ceil(Ncap/32), d, nbits]
    meta: object      # float16 [B, Hkv, Ncap, 2]
    m: int
    m_out: int
    nbits: int

    @property
    def Ncap(self) -> int:
        return int(self.bits.shape[2])


def code_tiles(Ncap: int) -> int:
    """Number of 32-position code tiles of a cache with capacity Ncap."""
    return (Ncap + 31) // 32


def alloc_cache(B: int, Hkv: int, Ncap: int, m: int, m_out: int, nbits: int = 2, d: int = 128,
                device="cuda") -> Cache:
    import torch
    W = (m + m_out) // 32
    return Cache(bits=torch.zeros((B, Hkv, Ncap, W), dtype=torch.int32, device=device),
                 norms=torch.zeros((B, Hkv, Ncap, 2), dtype=torch.float16, device=device),
                 codes=torch.zeros((B, Hkv, code_tiles(Ncap), d, nbits), dtype=torch.int32, device=device),
                 meta=torch.zeros((B, Hkv, Ncap, 2), dtype=torch.float16, device=device),
                 m=m, m_out=m_out, nbits=nbits)


def quantize_keys(K, S_in, S_out, outlier_idx, bits, norms, t0: int = 0, stream=None) -> None:
    """qjl_quantize_keys on torch tensors.  K [B, T, Hkv, d] (any strides with d contiguous)."""
    B, T, Hkv, d = K.shape
    if K.stride(3) != 1:
        raise ValueError("the d channels of K must be contiguous")
    _contiguous(S_in=S_in, S_out=S_out, outlier_idx=outlier_idx, bits=bits, norms=norms)
    m = S_in.shape[0]
    m_out = 0 if S_out is None else S_out.shape[0]
    n_out = 0 if outlier_idx is None or outlier_idx.numel() == 0 else outlier_idx.shape[1]
    _check(lib.qjl_quantize_keys(_ptr(K), _dtype_code(K), B, T, Hkv, d, K.stride(0), K.stride(1), K.stride(2),
                                 _ptr(S_in), m, _ptr(S_out) if m_out else 0, m_out,
                                 _ptr(outlier_idx) if n_out else 0, n_out, _ptr(bits), _ptr(norms),
                                 bits.shape[2], t0, _stream(stream)), "qjl_quantize_keys")


def quantize_values(V, nbits: int, codes, meta, t0: int = 0, stream=None) -> None:
    """qjl_quantize_values on torch tensors.  V [B, T, Hkv, d] (d contiguous); codes are the code
    tiles of a cache whose capacity is meta.shape[2]."""
    B, T, Hkv, d = V.shape
    if V.stride(3) != 1:
        raise ValueError("the d channels of V must be contiguous")
    _contiguous(codes=codes, meta=meta)
    Ncap = meta.shape[2]
    if codes.numel() * codes.element_size() < B * Hkv * code_tiles(Ncap) * d * nbits * 4:
        raise ValueError("codes is smaller than the code tiles of a cache of this capacity")
    _check(lib.qjl_quantize_values(_ptr(V), _dtype_code(V), B, T, Hkv, d, V.stride(0), V.stride(1), V.stride(2),
                                   nbits, _ptr(codes), _ptr(meta), Ncap, t0, _stream(stream)),
           "qjl_quantize_values")


def decode_workspace_size(B: int, Hq: int, Hkv: int, N: int, m: int, m_out: int, nsplit: int = 0,
                          d: int = 128) -> int:
    return int(lib.qjl_decode_workspace_size(B, Hq, Hkv, d, N, m, m_out, nsplit))


def decode_attention(Q, S_in, S_out, outlier_idx, bits, norms, N: int, out, *, codes=None, meta=None,
                     V_f32=None, nbits: int = 2, sm_scale: float = 0.0, estimator: int = 0, scores_dbg=None,
                     nsplit: int = 0, workspace=None, stream=None) -> None:
    """qjl_decode_attention on torch tensors.  Q [B, Hq, d] contiguous; out [B, Hq, d] fp32.
    estimator: QJL_EST_ONE_SIDED (0) or QJL_EST_TWO_SIDED (1)."""
    B, Hq, d = Q.shape
    if not Q.is_contiguous():
        raise ValueError("Q must be contiguous [B, Hq, d]")
    _contiguous(S_in=S_in, S_out=S_out, outlier_idx=outlier_idx, bits=bits, norms=norms, out=out, codes=codes,
                meta=meta, V_f32=V_f32, scores_dbg=scores_dbg, workspace=workspace)
    Hkv = bits.shape[1]
    m = S_in.shape[0]
    m_out = 0 if S_out is None else S_out.shape[0]
    n_out = 0 if outlier_idx is None or outlier_idx.numel() == 0 else outlier_idx.shape[1]
    vmode = QJL_V_F32 if V_f32 is not None else QJL_V_CODES
    if workspace is None:
        import torch
        workspace = torch.empty(max(1, decode_workspace_size(B, Hq, Hkv, N, m, m_out, nsplit, d)),
                                dtype=torch.uint8, device=Q.device)
    _check(lib.qjl_decode_attention(_ptr(Q), _dtype_code(Q), B, Hq, Hkv, d, N, _ptr(S_in), m,
                                    _ptr(S_out) if m_out else 0, m_out, _ptr(outlier_idx) if n_out else 0, n_out,
                                    _ptr(bits), _ptr(norms), bits.shape[2], vmode, _ptr(codes), _ptr(meta),
                                    _ptr(V_f32), nbits, sm_scale, estimator, _ptr(out), _ptr(scores_dbg), nsplit,
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "qjl_decode_attention")


def _step_args(Q, K_new, V_new, S_in, S_out, outlier_idx, cache: Cache, N: int, out, scores_dbg, workspace):
    """Shapes, checks and the pointer arguments shared by qjl_decode_step and its no-alloc variant."""
    B, Hq, d = Q.shape
    if not Q.is_contiguous():
        raise ValueError("Q must be contiguous [B, Hq, d]")
    for name, t in (("K_new", K_new), ("V_new", V_new)):
        if t.dim() != 4 or t.shape[1] != 1 or t.stride(3) != 1:
            raise ValueError(f"{name} must be [B, 1, Hkv, d] with the d channels contiguous")
        if t.dtype != Q.dtype:
            raise TypeError(f"{name} must have the dtype of Q")
    _contiguous(S_in=S_in, S_out=S_out, outlier_idx=outlier_idx, bits=cache.bits, norms=cache.norms,
                codes=cache.codes, meta=cache.meta, out=out, scores_dbg=scores_dbg, workspace=workspace)
    Hkv = cache.bits.shape[1]
    m = S_in.shape[0]
    m_out = 0 if S_out is None else S_out.shape[0]
    n_out = 0 if outlier_idx is None or outlier_idx.numel() == 0 else outlier_idx.shape[1]
    return (B, Hq, Hkv, d, m, m_out, n_out)


def decode_step(Q, K_new, V_new, S_in, S_out, outlier_idx, cache: Cache, N: int, out, *, sm_scale: float = 0.0,
                estimator: int = 0, scores_dbg=None, nsplit: int = 0, workspace=None, stream=None) -> None:
    """qjl_decode_step on torch tensors: append the new token (K_new, V_new [B, 1, Hkv, d], d contiguous)
    at position N - 1 of the cache, then decode Q [B, Hq, d] over the first N positions into out."""
    B, Hq, Hkv, d, m, m_out, n_out = _step_args(Q, K_new, V_new, S_in, S_out, outlier_idx, cache, N, out, scores_dbg,
                                                workspace)
    if workspace is None:
        import torch
        workspace = torch.empty(max(1, decode_workspace_size(B, Hq, Hkv, N, m, m_out, nsplit, d)),
                                dtype=torch.uint8, device=Q.device)
    _check(lib.qjl_decode_step(_ptr(Q), _ptr(K_new), _ptr(V_new), _dtype_code(Q), B, Hq, Hkv, d, N,
                               K_new.stride(0), K_new.stride(2), V_new.stride(0), V_new.stride(2),
                               _ptr(S_in), m, _ptr(S_out) if m_out else 0, m_out,
                               _ptr(outlier_idx) if n_out else 0, n_out, _ptr(cache.bits), _ptr(cache.norms),
                               _ptr(cache.codes), _ptr(cache.meta), cache.Ncap, cache.nbits, sm_scale, estimator, _ptr(out),
                               _ptr(scores_dbg), nsplit, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)), "qjl_decode_step")


def decode_step_no_alloc(Q, K_new, V_new, S_in, S_out, outlier_idx, cache: Cache, N: int, out, *,
                         sm_scale: float = 0.0, estimator: int = 0, scores_dbg=None, nsplit: int = 0,
                         stream=None) -> None:
    """qjl_decode_step_no_alloc on torch tensors: decode_step with the library's fixed device scratch as
    its workspace (NO_ALLOC_SCRATCH_BYTES per GPU); nothing is allocated, by the library or here.  Calls
    that overlap in time on one GPU race on the scratch."""
    B, Hq, Hkv, d, m, m_out, n_out = _step_args(Q, K_new, V_new, S_in, S_out, outlier_idx, cache, N, out, scores_dbg,
                                                None)
    _check(lib.qjl_decode_step_no_alloc(_ptr(Q), _ptr(K_new), _ptr(V_new), _dtype_code(Q), B, Hq, Hkv, d, N,
                                        K_new.stride(0), K_new.stride(2), V_new.stride(0), V_new.stride(2),
                                        _ptr(S_in), m, _ptr(S_out) if m_out else 0, m_out,
                                        _ptr(outlier_idx) if n_out else 0, n_out, _ptr(cache.bits), _ptr(cache.norms),
                                        _ptr(cache.codes), _ptr(cache.meta), cache.Ncap, cache.nbits, sm_scale, estimator,
                                        _ptr(out), _ptr(scores_dbg), nsplit, _stream(stream)),
           "qjl_decode_step_no_alloc")


def select_outliers(K, n_out: int, outlier_idx=None, *, workspace=None, stream=None):
    """qjl_select_outliers on torch tensors: K [B, T, Hkv, d] (d contiguous) -> int32 [Hkv, n_out],
    the channels with the largest mean |k_c| of each KV head, ascending."""
    import torch
    B, T, Hkv, d = K.shape
    if K.stride(3) != 1:
        raise ValueError("the d channels of K must be contiguous")
    if outlier_idx is None:
        outlier_idx = torch.empty((Hkv, n_out), dtype=torch.int32, device=K.device)
    _contiguous(outlier_idx=outlier_idx, workspace=workspace)
    if workspace is None:
        workspace = torch.empty(max(1, int(lib.qjl_select_outliers_workspace_size(B, T, Hkv, d))), dtype=torch.uint8,
                                device=K.device)
    _check(lib.qjl_select_outliers(_ptr(K), _dtype_code(K), B, T, Hkv, d, K.stride(0), K.stride(1), K.stride(2), n_out,
                                   _ptr(outlier_idx), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "qjl_select_outliers")
    return outlier_idx


def timer_enable(on: bool) -> None:
    _check(lib.qjl_timer_enable(1 if on else 0), "qjl_timer_enable")


def timer_read(kernel: str) -> tuple[int, float]:
    """(launches, total milliseconds) of one kernel since the last read; clears the record."""
    n = _i64(0)
    ms = ctypes.c_double(0.0)
    _check(lib.qjl_timer_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)), "qjl_timer_read")
    return int(n.value), float(ms.value)
