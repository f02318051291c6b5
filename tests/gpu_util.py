"""Shared helpers of the GPU parity tests: uploads, library calls, comparisons against the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle
import seeded_inputs as si


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_dev(x: np.ndarray, dtype: str, device="cuda"):
    """fp32 numpy array holding storage-type values -> device tensor of the storage type (exact)."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def inputs(w: si.Workload, T: int | None = None):
    oidx = si.outlier_channels(w)
    S_in, S_out = si.jl_matrices(w)
    K = si.keys(w, oidx, T)
    V = si.values(w, T)
    Q = si.queries(w)
    return dict(oidx=oidx, S_in=S_in, S_out=S_out, K=K, V=V, Q=Q)


def gpu_quantize_keys(qjl, w, K, S_in, S_out, oidx, Ncap=None, t0=0, Kdev=None):
    torch = torch_mod()
    B, T, Hkv, d = K.shape
    Ncap = T + t0 if Ncap is None else Ncap
    Kd = to_dev(K, w.dtype) if Kdev is None else Kdev
    cache = qjl.alloc_cache(B, Hkv, Ncap, w.m, w.m_out, w.nbits)
    qjl.quantize_keys(Kd, to_dev(S_in, w.dtype), to_dev(S_out, w.dtype) if w.m_out else None,
                      torch.from_numpy(oidx).cuda() if w.n_out else None, cache.bits, cache.norms, t0=t0)
    torch.cuda.synchronize()
    return cache


def bits_np(t, m: int, m_out: int):
    """Device sign-word rows -> numpy uint32 words in natural order (word w = projections 32w..32w+31)."""
    from bit_kv_cache_qjl_amd import layout
    return layout.bits_from_stored(t.cpu().numpy().view(np.uint32), m, m_out)


def bits_dev(words: np.ndarray, m: int, m_out: int):
    """Natural-order sign words (the oracle's) -> a device tensor in the library's row order."""
    from bit_kv_cache_qjl_amd import layout
    return torch_mod().from_numpy(np.ascontiguousarray(layout.bits_to_stored(words, m, m_out)).view(np.int32)).cuda()


def code_tiles_of_rows(rows: np.ndarray, nbits: int, ncap: int | None = None, d: int = 128) -> np.ndarray:
    """Oracle codes (per-token LSB-first bytes [..., n, d*nbits/8]) -> the library's code tiles."""
    from bit_kv_cache_qjl_amd import layout
    return layout.tiles_from_codes(oracle.unpack_codes(rows, nbits, d), nbits, ncap)


def code_rows_of_tiles(tiles, nbits: int, n: int) -> np.ndarray:
    """The library's code tiles (device tensor or array) -> oracle-format rows [..., n, d*nbits/8]."""
    from bit_kv_cache_qjl_amd import layout
    t = tiles.cpu().numpy() if hasattr(tiles, "cpu") else tiles
    return oracle.pack_codes(layout.codes_from_tiles(t, nbits, n), nbits)


def compare_bits(gpu_bits: np.ndarray, ref: dict, what: str, nbits_total: int):
    """Bit-exact except where the oracle flags |S k| < 1e-5 |k|; returns (mismatches, flagged)."""
    g = oracle.unpack_bits(gpu_bits, nbits_total)
    r = oracle.unpack_bits(ref["bits"], nbits_total)
    diff = g != r
    flagged = ref["near_zero"]
    bad = diff & ~flagged
    if bad.any():
        idx = np.argwhere(bad)[0]
        tok = tuple(idx[:-1])
        raise AssertionError(f"{what}: {int(bad.sum())} unflagged bit mismatches of {diff.size}; first at {tuple(idx)}; "
                             f"gpu words {gpu_bits[tok][:4]} oracle words {ref['bits'][tok][:4]}")
    log(f"  {what}: bits ok, {int(diff.sum())} mismatches all within {int(flagged.sum())} near-zero flags "
        f"of {diff.size}")
    return int(diff.sum()), int(flagged.sum())


def compare_norms(gpu: np.ndarray, ref: np.ndarray, what: str):
    """Within one fp16 ulp (norms are non-negative, so adjacent values differ by 1 in the pattern)."""
    a = gpu.view(np.uint16).astype(np.int64)
    b = ref.view(np.uint16).astype(np.int64)
    d = np.abs(a - b)
    assert d.max() <= 1, f"{what}: norm differs by {d.max()} fp16 ulps"
    log(f"  {what}: norms ok ({int((d == 1).sum())} of {d.size} one ulp apart)")


def score_tolerance(sq_in, sq_out, norms, m, m_out):
    """1e-3 relative to the estimator's magnitude scale sqrt(pi/2)(n_in |Sq_in|_1/m + n_out |Sq_out|_1/m_out)."""
    n_in = norms[:, 0].astype(np.float64)
    n_out = norms[:, 1].astype(np.float64)
    scale = n_in * np.abs(sq_in).sum() / m
    if m_out:
        scale = scale + n_out * np.abs(sq_out).sum() / m_out
    return 1e-3 * math.sqrt(math.pi / 2) * scale


def two_sided_tolerance(q, S_in, S_out, channels, norms, m, m_out):
    """1e-3 relative to the two-sided estimator's magnitude scale |q_in| n_in + |q_out| n_out, plus, for
    every query projection small enough that its sign may come out differently in the kernel's fp32
    sums (|S_j q| <= 1e-4 sum_c |S_jc q_c|), the full swing of that sign, 2 |q_part| n_part / m_part."""
    q = np.asarray(q, dtype=np.float64)
    mask = oracle.outlier_mask(q.shape[0], channels)
    qi, qo = q * (1.0 - mask), q * mask
    n_in = norms[:, 0].astype(np.float64)
    n_out = norms[:, 1].astype(np.float64)
    tol = 1e-3 * (np.linalg.norm(qi) * n_in + np.linalg.norm(qo) * n_out)
    amb_in = int(np.sum(np.abs(S_in @ qi) <= 1e-4 * (np.abs(S_in) @ np.abs(qi))))
    tol = tol + 2.0 * amb_in * np.linalg.norm(qi) * n_in / m
    if m_out:
        amb_out = int(np.sum(np.abs(S_out @ qo) <= 1e-4 * (np.abs(S_out) @ np.abs(qo))))
        tol = tol + 2.0 * amb_out * np.linalg.norm(qo) * n_out / m_out
    return tol


def run_decode(qjl, w, Q, S_in, S_out, oidx, cache_np: dict, N: int, *, nsplit=0, with_scores=True, V_f32=None,
               estimator=0, path=0):
    """Upload an oracle-built cache, run the library decode, return (out, scores) as numpy."""
    torch = torch_mod()
    B, Hq, d = Q.shape
    bits = bits_dev(cache_np["bits"], w.m, w.m_out)
    norms = torch.from_numpy(cache_np["norms"]).cuda()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    scores = torch.full((B, Hq, max(N, 1)), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
    kw = {}
    if V_f32 is not None:
        kw["V_f32"] = torch.from_numpy(np.ascontiguousarray(V_f32, dtype=np.float32)).cuda()
    else:
        tiles = code_tiles_of_rows(cache_np["codes"], w.nbits, bits.shape[2], w.d)
        kw["codes"] = torch.from_numpy(tiles.view(np.int32)).cuda()
        kw["meta"] = torch.from_numpy(cache_np["meta"]).cuda()
    qjl.decode_attention(to_dev(Q, w.dtype), to_dev(S_in, w.dtype), to_dev(S_out, w.dtype) if w.m_out else None,
                         torch.from_numpy(oidx).cuda() if w.n_out else None, bits, norms, N, out,
                         nbits=w.nbits, scores_dbg=scores, nsplit=nsplit, estimator=estimator, path=path, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (scores.cpu().numpy()[:, :, :N] if with_scores else None)


def device_cache_np(cache, w, N: int) -> dict:
    """The first N positions of a cache the library wrote, read back in the oracle's formats: natural-order
    sign words, fp16 norms, per-token packed code rows, fp16 (min, step)."""
    return {"bits": bits_np(cache.bits, w.m, w.m_out)[:, :, :N], "norms": cache.norms.cpu().numpy()[:, :, :N],
            "codes": code_rows_of_tiles(cache.codes, cache.nbits, N), "meta": cache.meta.cpu().numpy()[:, :, :N]}


def output_tolerance(meta_unit, nbits: int) -> float:
    """Max-abs output tolerance of one (sequence, KV head): 2e-3, or 1.25 * 2^-12 of the unit's largest
    value range R = L * step where that is larger (R > 6.5).  Both error sources of the output scale with
    the value range: the matrix-core path carries each softmax weight times step as three e4m3 pieces
    (relative residual <= 2^-12, so the value term can be off by 2^-12 R), and a score error moves
    weight between tokens whose values differ by up to R.  The 2e-3 bound is stated for the synthetic
    N(0, 1) values (ranges of 5 to 7); wider ranges keep the same relative bound."""
    if meta_unit is None or len(meta_unit) == 0:
        return 2e-3
    L = 2 ** nbits - 1
    rng = float(np.max(meta_unit[:, 1].astype(np.float64))) * L
    return max(2e-3, 1.25 * 2.0 ** -12 * rng)


def check_decode(w, Q, S_in, S_out, oidx, cache_np, N, out_gpu, scores_gpu, units, V_f32=None, what="",
                 estimator="one_sided"):
    """Compare sampled (b, hq) outputs (2e-3 max-abs; output_tolerance for wide value ranges) and scores
    (1e-3 of the estimator scale)."""
    ref = oracle.decode_attention(Q, S_in, S_out, oidx, cache_np["bits"], cache_np["norms"], N,
                                  codes=cache_np.get("codes"), meta=cache_np.get("meta"), V_f32=V_f32,
                                  nbits=w.nbits, units=units, estimator=estimator)
    worst_o, worst_s, worst_raw = 0.0, 0.0, 0.0
    g = w.Hq // w.Hkv
    for b, hq in units:
        h = hq // g
        err = np.abs(out_gpu[b, hq] - ref["out"][b, hq]).max()
        tol_o = 2e-3 if V_f32 is not None else output_tolerance(cache_np["meta"][b, h, :N], w.nbits)
        worst_o = max(worst_o, float(err) / tol_o * 2e-3)
        worst_raw = max(worst_raw, float(err))
        assert err <= tol_o, f"{what} out (b={b}, hq={hq}) max-abs {err:.3g} > {tol_o:.3g}"
        if scores_gpu is not None and N:
            channels = oidx[h] if oidx.size else []
            if estimator == "one_sided":
                sq_in, sq_out = oracle.project_query(Q[b, hq], S_in, S_out, channels)
                tol = score_tolerance(sq_in, sq_out, cache_np["norms"][b, h, :N], w.m, w.m_out)
            else:
                tol = two_sided_tolerance(Q[b, hq], S_in, S_out, channels, cache_np["norms"][b, h, :N], w.m, w.m_out)
            ds = np.abs(scores_gpu[b, hq] - ref["scores"][b, hq])
            ratio = float((ds / tol).max())
            worst_s = max(worst_s, ratio)
            assert ratio <= 1.0, f"{what} scores (b={b}, hq={hq}) exceed tolerance by x{ratio:.3g}"
    log(f"  {what}: out max-abs {worst_raw:.2e} ({worst_o / 2e-3:.2e} of its tolerance); worst score error "
        f"{worst_s:.2e} of tolerance")
    return worst_o, worst_s
