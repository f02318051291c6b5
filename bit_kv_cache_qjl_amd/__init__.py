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
QJL_PATH_AUTO = 0
QJL_PATH_MATRIX = 1
QJL_PATH_VECTOR = 2
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
                                     _i, _p, _p, _p, _i, _f, _i, _i, _p, _p, _i, _p, _sz, _p]
lib.qjl_decode_step.restype = _i
lib.qjl_decode_step.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64, _p, _i, _p, _i, _p, _i,
                                _p, _p, _p, _p, _i64, _i, _f, _i, _i, _p, _p, _i, _p, _sz, _p]
lib.qjl_decode_step_no_alloc.restype = _i
lib.qjl_decode_step_no_alloc.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64, _p, _i, _p, _i, _p,
                                         _i, _p, _p, _p, _p, _i64, _i, _f, _i, _i, _p, _p, _i, _p]
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


def _on_device(**tensors) -> None:
    """Every array the C ABI receives is device memory of one GPU."""
    devs = {t.device for t in tensors.values() if t is not None}
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a device (cuda) tensor, got {t.device}")
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(str(d) for d in devs)}")


def _check_tensor(name: str, t, dtype, ndim: int | None = None, shape: dict | None = None) -> None:
    """dtype, rank and the given {dimension: size} of one argument (TypeError / ValueError otherwise)."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    for dim, size in (shape or {}).items():
        if t.shape[dim] != size:
            raise ValueError(f"{name}: dimension {dim} must be {size}, got shape {tuple(t.shape)}")


def _sketch_args(S_in, S_out, outlier_idx, dtype, Hkv: int, d: int) -> tuple[int, int, int]:
    """JL matrices [m, d] / [m_out, d] of the key (or query) dtype and the int32 outlier list
    [Hkv, n_out]; returns (m, m_out, n_out)."""
    _check_tensor("S_in", S_in, dtype, 2, {1: d})
    m_out = 0
    if S_out is not None and S_out.numel():
        _check_tensor("S_out", S_out, dtype, 2, {1: d})
        m_out = int(S_out.shape[0])
    n_out = 0
    if outlier_idx is not None and outlier_idx.numel():
        import torch
        _check_tensor("outlier_idx", outlier_idx, torch.int32, 2, {0: Hkv})
        n_out = int(outlier_idx.shape[1])
    return int(S_in.shape[0]), m_out, n_out


def _key_cache_args(bits, norms, B: int, Hkv: int, m: int, m_out: int) -> int:
    """Sign words int32 [Bc, Hkv, Ncap, (m + m_out) / 32] and norms float16 [Bc, Hkv, Ncap, 2] with
    Bc >= B; returns Ncap."""
    import torch
    _check_tensor("bits", bits, torch.int32, 4, {1: Hkv, 3: (m + m_out) // 32})
    _check_tensor("norms", norms, torch.float16, 4, {0: bits.shape[0], 1: Hkv, 2: bits.shape[2], 3: 2})
    if bits.shape[0] < B:
        raise ValueError(f"the cache holds {bits.shape[0]} sequences, the call has {B}")
    return int(bits.shape[2])


def _value_cache_args(codes, meta, B: int, Hkv: int, nbits: int, d: int, Ncap: int | None = None) -> int:
    """Code tiles int32 [Bc, Hkv, ceil(Ncap/32), d, nbits] and meta float16 [Bc, Hkv, Ncap, 2] with
    Bc >= B; returns Ncap."""
    import torch
    if nbits not in (2, 3, 4):
        raise ValueError(f"nbits must be 2, 3 or 4, got {nbits}")
    Nc = int(meta.shape[2]) if meta.dim() == 4 else -1
    _check_tensor("meta", meta, torch.float16, 4, {1: Hkv, 3: 2})
    if Ncap is not None and Nc != Ncap:
        raise ValueError(f"meta holds {Nc} positions, the key cache {Ncap}")
    _check_tensor("codes", codes, torch.int32, 5, {0: meta.shape[0], 1: Hkv, 2: code_tiles(Nc), 3: d, 4: nbits})
    if meta.shape[0] < B:
        raise ValueError(f"the cache holds {meta.shape[0]} sequences, the call has {B}")
    return Nc


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
    """qjl_quantize_keys on torch tensors.  K [B, T, Hkv, d] (any strides with d contiguous); S_in, S_out
    of K's dtype; outlier_idx int32 [Hkv, n_out]; bits / norms the key cache (alloc_cache)."""
    if K.dim() != 4 or K.stride(3) != 1:
        raise ValueError("K must be [B, T, Hkv, d] with the d channels contiguous")
    B, T, Hkv, d = K.shape
    _contiguous(S_in=S_in, S_out=S_out, outlier_idx=outlier_idx, bits=bits, norms=norms)
    _on_device(K=K, S_in=S_in, S_out=S_out, outlier_idx=outlier_idx, bits=bits, norms=norms)
    m, m_out, n_out = _sketch_args(S_in, S_out, outlier_idx, K.dtype, Hkv, d)
    Ncap = _key_cache_args(bits, norms, B, Hkv, m, m_out)
    _check(lib.qjl_quantize_keys(_ptr(K), _dtype_code(K), B, T, Hkv, d, K.stride(0), K.stride(1), K.stride(2),
                                 _ptr(S_in), m, _ptr(S_out) if m_out else 0, m_out,
                                 _ptr(outlier_idx) if n_out else 0, n_out, _ptr(bits), _ptr(norms),
                                 Ncap, t0, _stream(stream)), "qjl_quantize_keys")


def quantize_values(V, nbits: int, codes, meta, t0: int = 0, stream=None) -> None:
    """qjl_quantize_values on torch tensors.  V [B, T, Hkv, d] (d contiguous); codes are the code
    tiles of a cache whose capacity is meta.shape[2] (alloc_cache with the same nbits)."""
    if V.dim() != 4 or V.stride(3) != 1:
        raise ValueError("V must be [B, T, Hkv, d] with the d channels contiguous")
    B, T, Hkv, d = V.shape
    _contiguous(codes=codes, meta=meta)
    _on_device(V=V, codes=codes, meta=meta)
    Ncap = _value_cache_args(codes, meta, B, Hkv, nbits, d)
    _check(lib.qjl_quantize_values(_ptr(V), _dtype_code(V), B, T, Hkv, d, V.stride(0), V.stride(1), V.stride(2),
                                   nbits, _ptr(codes), _ptr(meta), Ncap, t0, _stream(stream)),
           "qjl_quantize_values")


def decode_workspace_size(B: int, Hq: int, Hkv: int, N: int, m: int, m_out: int, nsplit: int = 0,
                          d: int = 128) -> int:
    return int(lib.qjl_decode_workspace_size(B, Hq, Hkv, d, N, m, m_out, nsplit))


def decode_attention(Q, S_in, S_out, outlier_idx, bits, norms, N: int, out, *, codes=None, meta=None,
                     V_f32=None, nbits: int | None = None, sm_scale: float = 0.0, estimator: int = 0, path: int = 0,
                     scores_dbg=None, nsplit: int = 0, workspace=None, stream=None) -> None:
    """qjl_decode_attention on torch tensors.  Q [B, Hq, d] contiguous; out [B, Hq, d] fp32; S_in, S_out
    of Q's dtype; values as code tiles + meta (nbits taken from the tiles when not given) or fp32 V_f32
    [B, Hkv, Ncap, d].  estimator: QJL_EST_ONE_SIDED (0) or QJL_EST_TWO_SIDED (1); path: QJL_PATH_AUTO (0),
    QJL_PATH_MATRIX (1, matrix cores) or QJL_PATH_VECTOR (2, vector units)."""
    import torch
    if Q.dim() != 3 or not Q.is_contiguous():
        raise ValueError("Q must be contiguous [B, Hq, d]")
    B, Hq, d = Q.shape
    _contiguous(S_in=S_in, S_out=S_out, outlier_idx=outlier_idx, bits=bits, norms=norms, out=out, codes=codes,
                meta=meta, V_f32=V_f32, scores_dbg=scores_dbg, workspace=workspace)
    _on_device(Q=Q, S_in=S_in, S_out=S_out, outlier_idx=outlier_idx, bits=bits, norms=norms, out=out, codes=codes,
               meta=meta, V_f32=V_f32, scores_dbg=scores_dbg, workspace=workspace)
    if bits.dim() != 4:
        raise ValueError(f"bits must be [B, Hkv, Ncap, W], got shape {tuple(bits.shape)}")
    Hkv = int(bits.shape[1])
    m, m_out, n_out = _sketch_args(S_in, S_out, outlier_idx, Q.dtype, Hkv, d)
    Ncap = _key_cache_args(bits, norms, B, Hkv, m, m_out)
    _check_tensor("out", out, torch.float32, 3, {0: B, 1: Hq, 2: d})
    if scores_dbg is not None:
        _check_tensor("scores_dbg", scores_dbg, torch.float32, 3, {0: B, 1: Hq})
        if N > 0 and scores_dbg.shape[2] != N:
            raise ValueError(f"scores_dbg must be [B, Hq, N] with N = {N}, got shape {tuple(scores_dbg.shape)}")
    if V_f32 is not None:
        vmode = QJL_V_F32
        _check_tensor("V_f32", V_f32, torch.float32, 4, {0: bits.shape[0], 1: Hkv, 2: Ncap, 3: d})
        nbits = 2 if nbits is None else nbits
    else:
        vmode = QJL_V_CODES
        if codes is None or meta is None:
            raise ValueError("values: give codes and meta, or V_f32")
        if nbits is None:
            nbits = int(codes.shape[-1])
        _value_cache_args(codes, meta, B, Hkv, nbits, d, Ncap)
    if workspace is None:
        workspace = torch.empty(max(1, decode_workspace_size(B, Hq, Hkv, N, m, m_out, nsplit, d)),
                                dtype=torch.uint8, device=Q.device)
    _check(lib.qjl_decode_attention(_ptr(Q), _dtype_code(Q), B, Hq, Hkv, d, N, _ptr(S_in), m,
                                    _ptr(S_out) if m_out else 0, m_out, _ptr(outlier_idx) if n_out else 0, n_out,
                                    _ptr(bits), _ptr(norms), Ncap, vmode, _ptr(codes), _ptr(meta),
                                    _ptr(V_f32), nbits, sm_scale, estimator, path, _ptr(out), _ptr(scores_dbg), nsplit,
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "qjl_decode_attention")


def _step_args(Q, K_new, V_new, S_in, S_out, outlier_idx, cache: Cache, N: int, out, scores_dbg, workspace):
    """Shapes, checks and the pointer arguments shared by qjl_decode_step and its no-alloc variant."""
    import torch
    if Q.dim() != 3 or not Q.is_contiguous():
        raise ValueError("Q must be contiguous [B, Hq, d]")
    B, Hq, d = Q.shape
    for name, t in (("K_new", K_new), ("V_new", V_new)):
        if t.dim() != 4 or t.shape[1] != 1 or t.stride(3) != 1:
            raise ValueError(f"{name} must be [B, 1, Hkv, d] with the d channels contiguous")
        if t.dtype != Q.dtype:
            raise TypeError(f"{name} must have the dtype of Q")
    _contiguous(S_in=S_in, S_out=S_out, outlier_idx=outlier_idx, bits=cache.bits, norms=cache.norms,
                codes=cache.codes, meta=cache.meta, out=out, scores_dbg=scores_dbg, workspace=workspace)
    _on_device(Q=Q, K_new=K_new, V_new=V_new, S_in=S_in, S_out=S_out, outlier_idx=outlier_idx, bits=cache.bits,
               norms=cache.norms, codes=cache.codes, meta=cache.meta, out=out, scores_dbg=scores_dbg,
               workspace=workspace)
    Hkv = int(cache.bits.shape[1])
    for name, t in (("K_new", K_new), ("V_new", V_new)):
        if t.shape[0] != B or t.shape[2] != Hkv or t.shape[3] != d:
            raise ValueError(f"{name} must be [B={B}, 1, Hkv={Hkv}, d={d}], got shape {tuple(t.shape)}")
    m, m_out, n_out = _sketch_args(S_in, S_out, outlier_idx, Q.dtype, Hkv, d)
    if (m, m_out) != (cache.m, cache.m_out):
        raise ValueError(f"S_in / S_out give m={m}, m_out={m_out}; the cache was built for {cache.m}, {cache.m_out}")
    Ncap = _key_cache_args(cache.bits, cache.norms, B, Hkv, m, m_out)
    _value_cache_args(cache.codes, cache.meta, B, Hkv, cache.nbits, d, Ncap)
    _check_tensor("out", out, torch.float32, 3, {0: B, 1: Hq, 2: d})
    if scores_dbg is not None:
        _check_tensor("scores_dbg", scores_dbg, torch.float32, 3, {0: B, 1: Hq, 2: N})
    return (B, Hq, Hkv, d, m, m_out, n_out)


def decode_step(Q, K_new, V_new, S_in, S_out, outlier_idx, cache: Cache, N: int, out, *, sm_scale: float = 0.0,
                estimator: int = 0, path: int = 0, scores_dbg=None, nsplit: int = 0, workspace=None,
                stream=None) -> None:
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
                               _ptr(cache.codes), _ptr(cache.meta), cache.Ncap, cache.nbits, sm_scale, estimator, path,
                               _ptr(out),
                               _ptr(scores_dbg), nsplit, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)), "qjl_decode_step")


def decode_step_no_alloc(Q, K_new, V_new, S_in, S_out, outlier_idx, cache: Cache, N: int, out, *,
                         sm_scale: float = 0.0, estimator: int = 0, path: int = 0, scores_dbg=None, nsplit: int = 0,
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
                                        path, _ptr(out), _ptr(scores_dbg), nsplit, _stream(stream)),
           "qjl_decode_step_no_alloc")


def select_outliers(K, n_out: int, outlier_idx=None, *, workspace=None, stream=None):
    """qjl_select_outliers on torch tensors: K [B, T, Hkv, d] (d contiguous) -> int32 [Hkv, n_out],
    the channels with the largest mean |k_c| of each KV head, ascending."""
    import torch
    if K.dim() != 4 or K.stride(3) != 1:
        raise ValueError("K must be [B, T, Hkv, d] with the d channels contiguous")
    B, T, Hkv, d = K.shape
    if outlier_idx is None:
        outlier_idx = torch.empty((Hkv, n_out), dtype=torch.int32, device=K.device)
    _contiguous(outlier_idx=outlier_idx, workspace=workspace)
    _on_device(K=K, outlier_idx=outlier_idx, workspace=workspace)
    _check_tensor("outlier_idx", outlier_idx, torch.int32, 2, {0: Hkv, 1: n_out})
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
