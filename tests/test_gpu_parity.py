"""GPU <-> oracle parity at sizes the oracle finishes in seconds (several tiles plus a ragged tail).

Bar: sign bits and value codes bit-exact, except sign bits whose projection
magnitude is below 1e-5 |k| (counted and reported); norms within one fp16 ulp; scores within 1e-3 of
the estimator's magnitude scale; attention outputs within 2e-3 max-abs.  Decode parity feeds both
sides the same oracle-built cache.
"""
import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import (bits_np, check_decode, code_rows_of_tiles, compare_bits, compare_norms, gpu_quantize_keys,
                      inputs, log, run_decode, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qjl = pytest.importorskip("bit_kv_cache_qjl_amd")

W = si.WORKLOADS

# scaled-down copies of every workload: same recipe and seed, small B / heads / context, ragged T
SCALED = {
    "tiny_fp32": W["tiny_fp32"],
    "llama2_7b_decode": W["llama2_7b_decode"].scaled(B=2, Hq=3, Hkv=3, N=1500),
    "llama3_8b_gqa_decode": W["llama3_8b_gqa_decode"].scaled(B=2, Hq=8, Hkv=2, N=1100),
    "prefill_quantize_64k": W["prefill_quantize_64k"].scaled(B=1, Hq=2, Hkv=2, N=1000),
    "llama31_70b_gqa_decode": W["llama31_70b_gqa_decode"].scaled(B=1, Hq=16, Hkv=2, N=777),
}
# a 1024-bit sketch (m = m_out = 512): decode takes the byte-table path for such wide sketches
WIDE = W["llama3_8b_gqa_decode"].scaled(B=2, Hq=6, Hkv=3, N=900, m=512, m_out=512)


@pytest.mark.parametrize("name", list(SCALED))
def test_quantize_keys_parity(name):
    w = SCALED[name]
    log(f"[quantize_keys] {name} B={w.B} T={w.N} Hkv={w.Hkv} m={w.m} m_out={w.m_out} n_out={w.n_out} {w.dtype}")
    x = inputs(w)
    cache = gpu_quantize_keys(qjl, w, x["K"], x["S_in"], x["S_out"], x["oidx"])
    ref = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    compare_bits(bits_np(cache.bits, w.m, w.m_out), ref, name, w.m + w.m_out)
    compare_norms(cache.norms.cpu().numpy(), ref["norms"], name)


@pytest.mark.parametrize("name,T,m,m_out", [
    ("llama2_7b_decode", 1, 256, 256),
    ("llama31_70b_gqa_decode", 5, 256, 256),
    ("prefill_quantize_64k", 16, 512, 512),
    ("prefill_quantize_64k", 17, 512, 512),
    ("llama3_8b_gqa_decode", 3, 128, 128),
    ("llama3_8b_gqa_decode", 2, 1024, 0),
])
def test_quantize_keys_small_append(name, T, m, m_out):
    """A few tokens per sequence (the decode-step append): the flattened-row kernel for T <= 16."""
    w = SCALED[name].scaled(N=T, m=m, m_out=m_out, n_out=SCALED[name].n_out if m_out else 0)
    log(f"[quantize_keys] small append {name} T={T} m={m} m_out={m_out} B={w.B} Hkv={w.Hkv}")
    x = inputs(w)
    cache = gpu_quantize_keys(qjl, w, x["K"], x["S_in"], x["S_out"], x["oidx"], Ncap=T + 9, t0=9)
    ref = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    bits = bits_np(cache.bits, w.m, w.m_out)
    compare_bits(bits[:, :, 9:], ref, f"append T={T}", w.m + w.m_out)
    compare_norms(cache.norms.cpu().numpy()[:, :, 9:], ref["norms"], f"append T={T}")
    assert not bits[:, :, :9].any()


@pytest.mark.parametrize("m,m_out", [(512, 512), (512, 0), (256, 256), (256, 0), (128, 128), (128, 0)])
def test_quantize_keys_sketch_shapes(m, m_out):
    """Every matrix-core sketch shape of the prefill quantizer (T > 16), three 32-token blocks and a
    ragged fourth per (sequence, KV head)."""
    base = SCALED["llama3_8b_gqa_decode"]
    w = base.scaled(B=2, Hq=2, Hkv=2, N=100, m=m, m_out=m_out, n_out=base.n_out if m_out else 0)
    log(f"[quantize_keys] sketch shape m={m} m_out={m_out} T={w.N}")
    x = inputs(w)
    cache = gpu_quantize_keys(qjl, w, x["K"], x["S_in"], x["S_out"], x["oidx"])
    ref = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    compare_bits(bits_np(cache.bits, w.m, w.m_out), ref, f"m={m} m_out={m_out}", w.m + w.m_out)
    compare_norms(cache.norms.cpu().numpy(), ref["norms"], f"m={m} m_out={m_out}")


def test_quantize_keys_append_offset_and_strides():
    """Write T tokens at t0 of a larger cache from a strided (non-contiguous) key view."""
    w = SCALED["llama2_7b_decode"].scaled(N=70)
    x = inputs(w)
    big = np.zeros((w.B, w.N, 2 * w.Hkv, w.d), dtype=np.float32)
    big[:, :, ::2, :] = x["K"]
    Kdev = to_dev(big, w.dtype)[:, :, ::2, :]
    assert not Kdev.is_contiguous()
    t0, Ncap = 37, 37 + w.N + 11
    log(f"[quantize_keys] strided view, t0={t0}, Ncap={Ncap}")
    cache = gpu_quantize_keys(qjl, w, x["K"], x["S_in"], x["S_out"], x["oidx"], Ncap=Ncap, t0=t0, Kdev=Kdev)
    ref = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    bits = bits_np(cache.bits, w.m, w.m_out)
    compare_bits(bits[:, :, t0:t0 + w.N], ref, "append", w.m + w.m_out)
    compare_norms(cache.norms.cpu().numpy()[:, :, t0:t0 + w.N], ref["norms"], "append")
    assert not bits[:, :, :t0].any() and not bits[:, :, t0 + w.N:].any(), "wrote outside [t0, t0 + T)"
    assert not cache.norms[:, :, :t0].any() and not cache.norms[:, :, t0 + w.N:].any()


def test_quantize_keys_special_keys():
    """Zero keys (every projection 0 -> all bits 1, norms 0), keys living only on the outlier
    channels (inlier bits all 1), and negated keys (complemented bits away from near-zero)."""
    w = SCALED["llama31_70b_gqa_decode"].scaled(N=64)
    x = inputs(w)
    K = x["K"].copy()
    K[:, :16] = 0.0
    only_out = np.zeros_like(K[:, 16:32])
    for h in range(w.Hkv):
        only_out[:, :, h, x["oidx"][h]] = K[:, 16:32, h, x["oidx"][h]]
    K[:, 16:32] = only_out
    K[:, 48:64] = -K[:, 32:48]
    log("[quantize_keys] special keys")
    cache = gpu_quantize_keys(qjl, w, K, x["S_in"], x["S_out"], x["oidx"])
    bits = bits_np(cache.bits, w.m, w.m_out)
    norms = cache.norms.cpu().numpy()
    assert np.all(bits[:, :, :16] == 0xFFFFFFFF) and np.all(norms[:, :, :16] == 0)
    assert np.all(bits[:, :, 16:32, : w.m // 32] == 0xFFFFFFFF) and np.all(norms[:, :, 16:32, 0] == 0)
    ref = oracle.quantize_keys(K, x["S_in"], x["S_out"], x["oidx"])
    compare_bits(bits, ref, "special", w.m + w.m_out)
    nz = ~(ref["near_zero"][:, :, 32:48] | ref["near_zero"][:, :, 48:64])
    a = oracle.unpack_bits(bits[:, :, 32:48], w.m + w.m_out)
    b = oracle.unpack_bits(bits[:, :, 48:64], w.m + w.m_out)
    assert np.all(a[nz] != b[nz])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_quantize_values_parity(dtype, nbits):
    w = SCALED["llama3_8b_gqa_decode"].scaled(dtype=dtype, nbits=nbits, N=333)
    log(f"[quantize_values] {dtype} nbits={nbits} B={w.B} T={w.N} Hkv={w.Hkv}")
    V = si.values(w)
    V[0, 0, 0, :] = 1.25                       # constant vector: step 0, all codes 0
    V[0, 1, 0, :5] = [3.0, -3.0, 0.0, 1.0, 2.0]
    torch_v = to_dev(V, dtype)
    cache = qjl.alloc_cache(w.B, w.Hkv, w.N + 3, w.m, w.m_out, nbits)
    qjl.quantize_values(torch_v, nbits, cache.codes, cache.meta, t0=3)
    torch.cuda.synchronize()
    ref = oracle.quantize_values(V, nbits)
    rows = code_rows_of_tiles(cache.codes, nbits, w.N + 3)
    meta = cache.meta.cpu().numpy()[:, :, 3:]
    np.testing.assert_array_equal(meta.view(np.uint16), ref["meta"].view(np.uint16))
    np.testing.assert_array_equal(rows[:, :, 3:], ref["codes"])
    assert not rows[:, :, :3].any(), "wrote codes before t0"
    assert not cache.meta[:, :, :3].any(), "wrote meta before t0"


@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_quantize_values_half_integer_quotients(nbits):
    """Values at and a few fp32 ulps around (k + 1/2) step, for steps that are not powers of two:
    the quotients (v - min) / step sit on or next to the rounding ties, where a code must come from
    the correctly rounded division and rint's ties to even."""
    L = (1 << nbits) - 1
    T, d = 96, 128
    rng = np.random.default_rng(7)
    V = np.zeros((1, T, 1, d), dtype=np.float32)
    for t in range(T):
        c = np.float32(rng.uniform(0.05, 3.0))
        step16 = np.float32(np.float16(np.float32(np.float32(L) * c) / np.float32(L)))
        row = [np.float32(0.0), np.float32(L) * c]
        for k in range(L):
            mid = np.float32((k + 0.5) * step16)
            for j in range(-3, 4):
                x = mid
                for _ in range(abs(j)):
                    x = np.nextafter(x, np.float32(np.inf if j > 0 else -np.inf), dtype=np.float32)
                row.append(x)
        row = np.array(row, dtype=np.float32)
        V[0, t, 0, :] = np.resize(row, d)
    log(f"[quantize_values] half-integer quotients nbits={nbits}")
    cache = qjl.alloc_cache(1, 1, T, 256, 0, nbits)
    qjl.quantize_values(to_dev(V, "f32"), nbits, cache.codes, cache.meta)
    torch.cuda.synchronize()
    ref = oracle.quantize_values(V, nbits)
    np.testing.assert_array_equal(cache.meta.cpu().numpy().view(np.uint16), ref["meta"].view(np.uint16))
    np.testing.assert_array_equal(code_rows_of_tiles(cache.codes, nbits, T), ref["codes"])


@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_quantize_values_appends_keep_neighbours(nbits):
    """Appends that start and end inside code tiles (single tokens, short runs, a run across tiles)
    merge into the tiles without touching other positions; the result equals one bulk quantize."""
    w = SCALED["llama2_7b_decode"].scaled(nbits=nbits, N=150)
    V = si.values(w)
    Vd = to_dev(V, w.dtype)
    cache = qjl.alloc_cache(w.B, w.Hkv, w.N, w.m, w.m_out, nbits)
    cache.codes.fill_(-1)                                  # garbage everywhere: only writes may change it
    log(f"[quantize_values] piecewise appends nbits={nbits}")
    for a, b in [(0, 1), (1, 5), (5, 31), (31, 33), (33, 34), (34, 97), (97, 149), (149, 150)]:
        qjl.quantize_values(Vd[:, a:b], nbits, cache.codes, cache.meta, t0=a)
    torch.cuda.synchronize()
    ref = oracle.quantize_values(V, nbits)
    rows = code_rows_of_tiles(cache.codes, nbits, w.N)
    np.testing.assert_array_equal(rows, ref["codes"])
    np.testing.assert_array_equal(cache.meta.cpu().numpy().view(np.uint16), ref["meta"].view(np.uint16))
    # the tail of the last tile (positions 150..159) was never appended: still all ones
    from bit_kv_cache_qjl_amd import layout
    tail = layout.codes_from_tiles(cache.codes.cpu().numpy(), nbits, 160)[:, :, 150:]
    assert np.all(tail == 2 ** nbits - 1)


@pytest.mark.parametrize("name", ["tiny_fp32", "llama2_7b_decode", "llama3_8b_gqa_decode", "llama31_70b_gqa_decode",
                                  "wide_sketch"])
@pytest.mark.parametrize("nsplit", [0, 1, 3])
def test_decode_parity(name, nsplit):
    w = WIDE if name == "wide_sketch" else SCALED[name]
    log(f"[decode] {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} nsplit={nsplit}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    cache = {"bits": kq["bits"], "norms": kq["norms"]}
    V_f32 = None
    if w.vmode == "codes":
        cache.update(oracle.quantize_values(x["V"], w.nbits))
    else:
        V_f32 = np.ascontiguousarray(x["V"].transpose(0, 2, 1, 3))       # [B, Hkv, N, d]
    out, scores = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, nsplit=nsplit, V_f32=V_f32)
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, out, scores, units, V_f32=V_f32, what=name)


@pytest.mark.parametrize("name", ["llama2_7b_decode", "llama3_8b_gqa_decode", "llama31_70b_gqa_decode"])
@pytest.mark.parametrize("nsplit", [0, 3])
@pytest.mark.parametrize("nbits", [3, 4])
def test_decode_parity_wider_values(name, nsplit, nbits):
    """3- and 4-bit token-wise value codes (a 2-bit plane plus a high-bit plane, or two 2-bit planes, on
    the matrix cores)."""
    w = SCALED[name].scaled(nbits=nbits)
    log(f"[decode {nbits}-bit] {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} nsplit={nsplit}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    cache = {"bits": kq["bits"], "norms": kq["norms"], **oracle.quantize_values(x["V"], nbits)}
    out, scores = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, nsplit=nsplit)
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, out, scores, units, what=f"{name} {nbits}-bit")


@pytest.mark.parametrize("name", ["tiny_fp32", "llama2_7b_decode", "llama3_8b_gqa_decode", "llama31_70b_gqa_decode",
                                  "wide_sketch", "fp32_queries"])
@pytest.mark.parametrize("nsplit", [0, 3])
def test_decode_parity_two_sided(name, nsplit):
    """The two-sided estimator (query reduced to its signs too) on every query-projection kernel: the
    matrix-core prologue (bf16), the fp32 projection of the matrix-core path, and the VALU path
    (fp32 values, and a sketch wider than the matrix-core shapes)."""
    if name == "wide_sketch":
        w = WIDE
    elif name == "fp32_queries":
        w = SCALED["llama3_8b_gqa_decode"].scaled(dtype="f32")
    else:
        w = SCALED[name]
    log(f"[decode two-sided] {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} nsplit={nsplit}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    cache = {"bits": kq["bits"], "norms": kq["norms"]}
    V_f32 = None
    if w.vmode == "codes":
        cache.update(oracle.quantize_values(x["V"], w.nbits))
    else:
        V_f32 = np.ascontiguousarray(x["V"].transpose(0, 2, 1, 3))
    out, scores = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, nsplit=nsplit, V_f32=V_f32,
                             estimator=qjl.QJL_EST_TWO_SIDED)
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, out, scores, units, V_f32=V_f32,
                 what=f"{name} two-sided", estimator="two_sided")


def test_decode_rotate_then_sign():
    """Rotate-then-sign keys: m = d = 128, no outlier copy, S_in = sqrt(2d/pi) R for an orthogonal R
    (stored in bf16); the one-sided decode then scores <R q, |k| sign(R k)/sqrt(d)>, which the oracle
    computes from R directly (R = S_in / sqrt(2d/pi), the exact rotation the kernels' signs come from)."""
    w = SCALED["llama3_8b_gqa_decode"].scaled(m=128, m_out=0, n_out=0, N=700)
    log(f"[decode rotate-then-sign] B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N}")
    x = inputs(w)
    alpha = math.sqrt(2 * w.d / math.pi)
    S = si.round_bf16((alpha * si.random_rotation(17, w.d)).astype(np.float32))
    R = S.astype(np.float64) / alpha
    oidx = np.zeros((w.Hkv, 0), np.int32)
    empty = np.zeros((0, w.d), np.float32)
    kq = oracle.quantize_keys(x["K"], S, empty, oidx)
    cache = {"bits": kq["bits"], "norms": kq["norms"], **oracle.quantize_values(x["V"], w.nbits)}
    out, scores = run_decode(qjl, w, x["Q"], S, empty, oidx, cache, w.N)
    g = w.Hq // w.Hkv
    worst = 0.0
    for b in range(w.B):
        for hq in range(w.Hq):
            h = hq // g
            K = x["K"][b, :, h]
            ref = oracle.rotate_sign_scores(x["Q"][b, hq], K, R)
            # the kernels use the fp16-rounded key norm: tolerance 1e-3 of the scale plus the norm rounding
            scale = np.linalg.norm(K, axis=1) * np.abs(R @ x["Q"][b, hq]).sum() / math.sqrt(w.d)
            err = np.abs(scores[b, hq] - ref)
            worst = max(worst, float((err / scale).max()))
            assert np.all(err <= (1e-3 + 2 ** -11) * scale), f"rotate-then-sign scores (b={b}, hq={hq})"
    log(f"  rotate-then-sign: worst score error {worst:.2e} of the scale")
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], S, empty, oidx, cache, w.N, out, scores, units, what="rotate-then-sign")


@pytest.mark.parametrize("N", [0, 1, 511, 513])
def test_decode_edge_lengths(N):
    w = SCALED["llama3_8b_gqa_decode"].scaled(N=600)
    log(f"[decode] edge N={N}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    cache = {"bits": kq["bits"], "norms": kq["norms"], **oracle.quantize_values(x["V"], w.nbits)}
    out, scores = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, N, nsplit=0)
    if N == 0:
        assert np.all(out == 0)
        return
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, N, out, scores, units, what=f"N={N}")
    if N == 1:
        vhat = oracle.dequantize_value_vectors(oracle.unpack_codes(cache["codes"][:, :, :1], 2, w.d), cache["meta"][:, :, :1])
        g = w.Hq // w.Hkv
        for b in range(w.B):
            for hq in range(w.Hq):
                np.testing.assert_allclose(out[b, hq], vhat[b, hq // g, 0], atol=2e-3)


def test_decode_many_splits_and_equal_scores():
    """More splits than tiles (empty chunks) and a cache whose keys are all equal (uniform softmax:
    the output is the mean of the dequantized values)."""
    w = SCALED["llama2_7b_decode"].scaled(N=700)
    x = inputs(w)
    K = np.repeat(x["K"][:, :1], w.N, axis=1)
    kq = oracle.quantize_keys(K, x["S_in"], x["S_out"], x["oidx"])
    cache = {"bits": kq["bits"], "norms": kq["norms"], **oracle.quantize_values(x["V"], w.nbits)}
    log("[decode] equal keys, nsplit=40")
    out, scores = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, nsplit=40)
    vhat = oracle.dequantize_value_vectors(oracle.unpack_codes(cache["codes"], 2, w.d), cache["meta"])
    for b in range(w.B):
        for hq in range(w.Hq):
            np.testing.assert_allclose(out[b, hq], vhat[b, hq].mean(axis=0), atol=2e-3)
            assert np.all(scores[b, hq] == scores[b, hq, 0])


def test_decode_step_append_then_attend():
    """The serving step: quantize the new token's key and value into slot N-1 of a cache built by
    prefill, then attend over all N tokens; compared with the oracle on the same inputs."""
    w = SCALED["llama31_70b_gqa_decode"].scaled(N=900)
    x = inputs(w)
    N = w.N
    log("[pipeline] prefill N-1 tokens, append 1, decode")
    cache = qjl.alloc_cache(w.B, w.Hkv, N, w.m, w.m_out, w.nbits)
    Kd, Vd = to_dev(x["K"], w.dtype), to_dev(x["V"], w.dtype)
    S_in, S_out = to_dev(x["S_in"], w.dtype), to_dev(x["S_out"], w.dtype)
    oidx = torch.from_numpy(x["oidx"]).cuda()
    qjl.quantize_keys(Kd[:, : N - 1], S_in, S_out, oidx, cache.bits, cache.norms, t0=0)
    qjl.quantize_values(Vd[:, : N - 1], w.nbits, cache.codes, cache.meta, t0=0)
    qjl.quantize_keys(Kd[:, N - 1:], S_in, S_out, oidx, cache.bits, cache.norms, t0=N - 1)
    qjl.quantize_values(Vd[:, N - 1:], w.nbits, cache.codes, cache.meta, t0=N - 1)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    qjl.decode_attention(to_dev(x["Q"], w.dtype), S_in, S_out, oidx, cache.bits, cache.norms, N, out,
                         codes=cache.codes, meta=cache.meta, nbits=w.nbits)
    torch.cuda.synchronize()
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    vq = oracle.quantize_values(x["V"], w.nbits)
    compare_bits(bits_np(cache.bits, w.m, w.m_out), kq, "pipeline", w.m + w.m_out)
    np.testing.assert_array_equal(code_rows_of_tiles(cache.codes, w.nbits, N), vq["codes"])
    # decode input must be identical on both sides: use the oracle cache where a near-zero bit differs
    gbits = bits_np(cache.bits, w.m, w.m_out)
    if np.array_equal(gbits, kq["bits"]) and np.array_equal(cache.norms.cpu().numpy().view(np.uint16),
                                                             kq["norms"].view(np.uint16)):
        cache_np = {"bits": kq["bits"], "norms": kq["norms"], **vq}
        units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
        check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache_np, N, out.cpu().numpy(), None, units,
                     what="pipeline")
    else:
        log("  pipeline: GPU cache differs from the oracle's in near-zero bits or a norm ulp; "
            "decode parity re-run on the oracle cache")
        cache_np = {"bits": kq["bits"], "norms": kq["norms"], **vq}
        o2, s2 = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache_np, N)
        units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
        check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache_np, N, o2, s2, units, what="pipeline")


# ----------------------------------------------------------------------------- sketch shapes of the
# VGPR-stationary key quantizer (T > 16 with m not in {128, 256, 512} or m_out not in {0, m}): one, two
# and four 32-projection tiles per wave, outlier sketches narrower and wider than the inlier one

@pytest.mark.parametrize("m,m_out", [(256, 128), (128, 256), (384, 384), (640, 0), (1024, 0), (512, 384)])
def test_quantize_keys_vgpr_kernel_shapes(m, m_out):
    base = SCALED["llama31_70b_gqa_decode"]
    w = base.scaled(B=2, Hq=2, Hkv=2, N=100, m=m, m_out=m_out, n_out=base.n_out if m_out else 0)
    log(f"[quantize_keys] VGPR kernel m={m} m_out={m_out} T={w.N} (64-token chunk + ragged 36), t0=5")
    x = inputs(w)
    cache = gpu_quantize_keys(qjl, w, x["K"], x["S_in"], x["S_out"], x["oidx"], Ncap=w.N + 12, t0=5)
    ref = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    bits = bits_np(cache.bits, w.m, w.m_out)
    compare_bits(bits[:, :, 5:5 + w.N], ref, f"m={m} m_out={m_out}", w.m + w.m_out)
    compare_norms(cache.norms.cpu().numpy()[:, :, 5:5 + w.N], ref["norms"], f"m={m} m_out={m_out}")
    assert not bits[:, :, :5].any() and not bits[:, :, 5 + w.N:].any(), "wrote outside [t0, t0 + T)"


# ----------------------------------------------------------------------------- outlier lists in any order

def _shuffled(oidx: np.ndarray, seed: int) -> np.ndarray:
    """The same channel sets, each KV head's list in a seeded random order (never the sorted one)."""
    rng = np.random.default_rng(seed)
    out = oidx.copy()
    for h in range(out.shape[0]):
        while out.shape[1] > 1 and np.all(np.diff(out[h]) > 0):
            out[h] = rng.permutation(oidx[h])
    return out


@pytest.mark.parametrize("kernel,T,m,m_out", [("lds", 100, 256, 256), ("rows", 3, 256, 256), ("vgpr", 100, 384, 384),
                                              ("lds_512", 70, 512, 512)])
def test_quantize_keys_unsorted_outlier_lists(kernel, T, m, m_out):
    w = SCALED["llama31_70b_gqa_decode"].scaled(B=2, Hq=2, Hkv=2, N=T, m=m, m_out=m_out)
    x = inputs(w)
    oidx = _shuffled(x["oidx"], 5)
    log(f"[quantize_keys] unsorted outlier lists ({kernel}) {oidx.tolist()}")
    cache = gpu_quantize_keys(qjl, w, x["K"], x["S_in"], x["S_out"], oidx)
    ref = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], oidx)
    compare_bits(bits_np(cache.bits, w.m, w.m_out), ref, f"unsorted {kernel}", w.m + w.m_out)
    compare_norms(cache.norms.cpu().numpy(), ref["norms"], f"unsorted {kernel}")


@pytest.mark.parametrize("name", ["llama31_70b_gqa_decode", "llama3_8b_gqa_decode", "fp32_queries", "wide_sketch"])
def test_decode_unsorted_outlier_lists(name):
    """The matrix-core prologue (bf16), the fp32 query projection and the byte-table path (1024-bit
    sketch) with each KV head's outlier list in a random order."""
    if name == "wide_sketch":
        w = WIDE
    elif name == "fp32_queries":
        w = SCALED["llama3_8b_gqa_decode"].scaled(dtype="f32")
    else:
        w = SCALED[name]
    x = inputs(w)
    oidx = _shuffled(x["oidx"], 9)
    log(f"[decode] unsorted outlier lists {name}")
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], oidx)
    cache = {"bits": kq["bits"], "norms": kq["norms"], **oracle.quantize_values(x["V"], w.nbits)}
    out, scores = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], oidx, cache, w.N)
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], oidx, cache, w.N, out, scores, units, what=f"unsorted {name}")


# ----------------------------------------------------------------------------- values with outlier channels

@pytest.mark.parametrize("nbits", [2, 3, 4])
@pytest.mark.parametrize("scale", [20.0, 50.0])
def test_decode_values_with_outlier_channels(nbits, scale):
    """Value vectors with three channels scaled x20 / x50 (value ranges of ~60 / ~150 instead of ~6):
    codes exact, and the decode output within output_tolerance, which grows with the value range (the
    page's outlier example spans 99.4: "Why Outliers Destroy Quantization")."""
    w = SCALED["llama31_70b_gqa_decode"].scaled(N=600, nbits=nbits)
    x = inputs(w)
    V = x["V"].copy()
    V[:, :, :, [7, 70, 101]] *= np.float32(scale)
    V = si.round_bf16(V)
    vq = oracle.quantize_values(V, nbits)
    # the library's codes for these values equal the oracle's
    vd = qjl.alloc_cache(w.B, w.Hkv, w.N, w.m, w.m_out, nbits)
    qjl.quantize_values(to_dev(V, w.dtype), nbits, vd.codes, vd.meta)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(code_rows_of_tiles(vd.codes, nbits, w.N), vq["codes"])
    np.testing.assert_array_equal(vd.meta.cpu().numpy().view(np.uint16), vq["meta"].view(np.uint16))
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    cache = {"bits": kq["bits"], "norms": kq["norms"], **vq}
    rng_max = float(vq["meta"][..., 1].astype(np.float64).max()) * (2 ** nbits - 1)
    log(f"[decode] values with x{scale:g} channels, {nbits}-bit: largest value range {rng_max:.1f}")
    for nsplit in (0, 3):
        out, scores = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, nsplit=nsplit)
        units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
        check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, out, scores, units,
                     what=f"x{scale:g} values {nbits}-bit nsplit={nsplit}")


# ----------------------------------------------------------------------------- the two decode paths

@pytest.mark.parametrize("name", ["llama2_7b_decode", "llama3_8b_gqa_decode", "llama31_70b_gqa_decode"])
@pytest.mark.parametrize("nsplit", [0, 3])
@pytest.mark.parametrize("estimator", ["one_sided", "two_sided"])
def test_decode_parity_vector_path(name, nsplit, estimator):
    """The vector-unit decode (byte tables of the projected query, fp16 value weights) forced on the
    2-bit matrix-core shapes, against the oracle."""
    w = SCALED[name]
    log(f"[decode vector path] {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} nsplit={nsplit} {estimator}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    cache = {"bits": kq["bits"], "norms": kq["norms"], **oracle.quantize_values(x["V"], w.nbits)}
    est = qjl.QJL_EST_ONE_SIDED if estimator == "one_sided" else qjl.QJL_EST_TWO_SIDED
    out, scores = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, nsplit=nsplit,
                             estimator=est, path=qjl.QJL_PATH_VECTOR)
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, out, scores, units,
                 what=f"{name} vector path", estimator=estimator)


def test_decode_paths_refuse_what_they_cannot_run():
    w = SCALED["llama3_8b_gqa_decode"]
    x = inputs(w.scaled(N=64))
    kq = oracle.quantize_keys(x["K"][:, :64], x["S_in"], x["S_out"], x["oidx"])
    cache = {"bits": kq["bits"], "norms": kq["norms"], **oracle.quantize_values(x["V"][:, :64], 3)}
    with pytest.raises(qjl.QJLError) as e:
        run_decode(qjl, w.scaled(nbits=3), x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, 64, path=qjl.QJL_PATH_VECTOR)
    assert e.value.status == qjl.QJL_ERR_UNSUPPORTED


# ----------------------------------------------------------------------------- eight-wave decode (g > 4)

@pytest.mark.parametrize("m,m_out", [(256, 256), (512, 0), (128, 0)])
@pytest.mark.parametrize("N,nsplit", [(777, 0), (1500, 3), (2049, 1), (300, 40)])
@pytest.mark.parametrize("with_scores", [True, False])
def test_decode_parity_eight_wave_shapes(m, m_out, N, nsplit, with_scores):
    """Query groups larger than 4 with 2-bit codes take the eight-wave kernel (block data staged in LDS
    by loads that write LDS directly): every sketch shape it serves, ragged contexts, one chunk, several
    and more chunks than blocks, with and without the score output (the benchmark's launch)."""
    base = SCALED["llama31_70b_gqa_decode"]
    w = base.scaled(B=2, Hq=16, Hkv=2, N=N, m=m, m_out=m_out, n_out=base.n_out if m_out else 0)
    log(f"[decode eight-wave] m={m} m_out={m_out} N={N} nsplit={nsplit} scores={with_scores}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    cache = {"bits": kq["bits"], "norms": kq["norms"], **oracle.quantize_values(x["V"], w.nbits)}
    out, scores = run_decode(qjl, w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, nsplit=nsplit,
                             with_scores=with_scores)
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache, w.N, out, scores, units,
                 what=f"eight-wave m={m} m_out={m_out} N={N}")
