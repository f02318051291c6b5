"""Seeded synthetic inputs for the 1-bit QJL KV-cache path.

This module is shared by the CPU oracle tests, the GPU parity tests and the benchmark. It holds none
of the method's arithmetic: it only draws Gaussian numbers, picks outlier channel sets and rounds the
draws to the device storage type (bfloat16, round-to-nearest-even), so that every consumer sees the
very same array values.

Input recipe (stands in for the long-context model workloads that the QJL summary evaluates on,
"Experimental setup" of "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with Zero
Overhead"; no dataset or trained weight is used):
  * keys, values and queries are i.i.d. N(0, 1);
  * a key's outlier channels (a few per KV head, drawn per head and sorted) are multiplied by the
    workload's factor (x20 / x30 / x50, inside the "10-100x" range of "The Third Problem: Magnitude
    Outliers" in "Why Compressing the KV Cache Is Hard"); queries and values carry no outliers;
  * the JL matrices S_in (m x d) and S_out (m_out x d) are i.i.d. N(0, 1) (the Gaussian JL transform of
    the QJL summary, "Approach"); they are inputs, never drawn inside the method;
  * bf16 workloads round every array to bfloat16 (RNE); the fp32 workload keeps float32.

Streams: one numpy PCG64 SeedSequence per workload (master seed), with spawn keys
(stream, b, h) so that any (batch, head) slice can be regenerated alone.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

# stream ids of the spawn keys
_S_IN, _S_OUT, _OUTLIERS, _KEYS, _VALUES, _QUERIES = range(6)


@dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one workload."""

    name: str
    B: int              # batch (sequences)
    Hq: int             # query heads
    Hkv: int            # KV heads
    d: int              # head dimension
    m: int              # JL dimension of the inlier sketch
    m_out: int          # JL dimension of the outlier sketch (0 = no outlier split)
    n_out: int          # outlier channels per KV head
    outlier_scale: float
    N: int              # context length (decode) / tokens quantized (prefill)
    dtype: str          # "bf16" or "f32" storage of K, V, Q and S
    vmode: str          # "codes" (token-wise quantized values) or "f32" (values kept as fp32)
    nbits: int          # value code width
    seed: int

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    def scaled(self, **kw) -> "Workload":
        """Same recipe and seed with some sizes changed (for scaled-down parity cases)."""
        return replace(self, **kw)


WORKLOADS = {
    # 1 head, d=128, m=256, 1024 keys, fp32 everything, values unquantized, no outlier split.
    "tiny_fp32": Workload("tiny_fp32", B=1, Hq=1, Hkv=1, d=128, m=256, m_out=0, n_out=0,
                          outlier_scale=1.0, N=1024, dtype="f32", vmode="f32", nbits=2, seed=1000),
    # Llama-2-7B-shaped one-layer decode: 32 heads MHA, batch 8, context 32768.
    "llama2_7b_decode": Workload("llama2_7b_decode", B=8, Hq=32, Hkv=32, d=128, m=256, m_out=256,
                                 n_out=4, outlier_scale=20.0, N=32768, dtype="bf16", vmode="codes",
                                 nbits=2, seed=1001),
    # Llama-3-8B-shaped GQA decode: 32 query / 8 KV heads, batch 4, context 131072.
    "llama3_8b_gqa_decode": Workload("llama3_8b_gqa_decode", B=4, Hq=32, Hkv=8, d=128, m=256,
                                     m_out=256, n_out=3, outlier_scale=30.0, N=131072, dtype="bf16",
                                     vmode="codes", nbits=2, seed=1002),
    # Prefill key-quantize stream: 65536 tokens x 8 KV heads, m = m_out = 512.
    "prefill_quantize_64k": Workload("prefill_quantize_64k", B=1, Hq=8, Hkv=8, d=128, m=512,
                                     m_out=512, n_out=4, outlier_scale=20.0, N=65536, dtype="bf16",
                                     vmode="codes", nbits=2, seed=1003),
    # Llama-3.1-70B-shaped one-layer decode: 64 query / 8 KV heads, batch 16, context 131072.
    "llama31_70b_gqa_decode": Workload("llama31_70b_gqa_decode", B=16, Hq=64, Hkv=8, d=128, m=256,
                                       m_out=256, n_out=5, outlier_scale=50.0, N=131072,
                                       dtype="bf16", vmode="codes", nbits=2, seed=1004),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 holding the bf16 value."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = (u + (((u >> 16) & 1) + np.uint32(0x7FFF))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bfloat16 storage (uint16) of an array whose values are already bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array is not bf16-exact")
    return (u >> 16).astype(np.uint16)


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def jl_matrices(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """S_in [m, d] and S_out [m_out, d], i.i.d. N(0, 1), in the workload's storage type (as fp32)."""
    s_in = _to_dtype(_rng(w.seed, _S_IN).standard_normal((w.m, w.d), dtype=np.float32), w.dtype)
    s_out = _to_dtype(_rng(w.seed, _S_OUT).standard_normal((w.m_out, w.d), dtype=np.float32), w.dtype)
    return s_in, s_out


def outlier_channels(w: Workload) -> np.ndarray:
    """[Hkv, n_out] int32: distinct channels per KV head, sorted."""
    rng = _rng(w.seed, _OUTLIERS)
    out = np.zeros((w.Hkv, w.n_out), dtype=np.int32)
    for h in range(w.Hkv):
        out[h] = np.sort(rng.choice(w.d, size=w.n_out, replace=False))
    return out


def key_slice(w: Workload, b: int, h: int, outliers: np.ndarray, T: int | None = None) -> np.ndarray:
    """Keys of sequence b, KV head h: [T, d] fp32 holding storage-type values."""
    T = w.N if T is None else T
    k = _rng(w.seed, _KEYS, b, h).standard_normal((T, w.d), dtype=np.float32)
    if w.n_out:
        k[:, outliers[h]] *= np.float32(w.outlier_scale)
    return _to_dtype(k, w.dtype)


def value_slice(w: Workload, b: int, h: int, T: int | None = None) -> np.ndarray:
    """Values of sequence b, KV head h: [T, d] fp32 holding storage-type values."""
    T = w.N if T is None else T
    return _to_dtype(_rng(w.seed, _VALUES, b, h).standard_normal((T, w.d), dtype=np.float32), w.dtype)


def queries(w: Workload) -> np.ndarray:
    """One decode query per sequence and query head: [B, Hq, d]."""
    return _to_dtype(_rng(w.seed, _QUERIES).standard_normal((w.B, w.Hq, w.d), dtype=np.float32), w.dtype)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def keys(w: Workload, outliers: np.ndarray, T: int | None = None) -> np.ndarray:
    """All keys in the model layout [B, T, Hkv, d] (fp32 array holding storage-type values)."""
    T = w.N if T is None else T
    K = np.empty((w.B, T, w.Hkv, w.d), dtype=np.float32)

    def fill(bh):
        b, h = bh
        K[b, :, h, :] = key_slice(w, b, h, outliers, T)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, [(b, h) for b in range(w.B) for h in range(w.Hkv)]))
    return K


def values(w: Workload, T: int | None = None) -> np.ndarray:
    """All values in the model layout [B, T, Hkv, d]."""
    T = w.N if T is None else T
    V = np.empty((w.B, T, w.Hkv, w.d), dtype=np.float32)

    def fill(bh):
        b, h = bh
        V[b, :, h, :] = value_slice(w, b, h, T)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, [(b, h) for b in range(w.B) for h in range(w.Hkv)]))
    return V


def gaussian(seed: int, shape, *key: int) -> np.ndarray:
    """Plain fp64 N(0, 1) draws for statistical tests (no storage rounding)."""
    return _rng(seed, 99, *key).standard_normal(shape)


def random_rotation(seed: int, d: int, *key: int) -> np.ndarray:
    """A random orthogonal d x d matrix (fp64): the QR factor of a Gaussian draw, column signs fixed
    by the diagonal of R so that the draw is uniform over the orthogonal group."""
    q, r = np.linalg.qr(_rng(seed, 98, *key).standard_normal((d, d)))
    return q * np.sign(np.diag(r))[None, :]
