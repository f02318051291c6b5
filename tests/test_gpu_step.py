"""GPU parity of the decode step (qjl_decode_step): append the new token at position N - 1, then decode.

The cache prefix (positions 0 .. N-2) is the oracle's own cache uploaded to the device; the step
writes position N - 1 and attends over N positions.  Checks: the appended row against the oracle
(sign bits exact except near-zero projections, norms within one fp16 ulp, codes and meta exact),
positions past N untouched, the fused path against the three separate calls, and the output
against the oracle (2e-3 max-abs) run on the cache the GPU wrote (so both sides attend over identical
inputs even where the appended row differs from the oracle's in a near-zero bit or a norm ulp).
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import bits_dev, bits_np, check_decode, compare_bits, compare_norms, device_cache_np, inputs, log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qjl = pytest.importorskip("bit_kv_cache_qjl_amd")
from bit_kv_cache_qjl_amd import layout  # noqa: E402

W = si.WORKLOADS
L3 = W["llama3_8b_gqa_decode"].scaled(B=2, Hq=8, Hkv=2, N=1100)
CASES = {
    "llama2_mha": W["llama2_7b_decode"].scaled(B=2, Hq=3, Hkv=3, N=1500),
    "llama3_gqa": L3,
    "llama31_70b_gqa": W["llama31_70b_gqa_decode"].scaled(B=1, Hq=16, Hkv=2, N=777),
    "group16": L3.scaled(B=1, Hq=32, Hkv=2, N=300),            # 17 projected vectors: two passes
    "m128_out128": L3.scaled(m=128, m_out=128, N=257),
    "m128_no_outliers": L3.scaled(m=128, m_out=0, n_out=0, N=64),
    "m256_no_outliers": L3.scaled(m=256, m_out=0, n_out=0, N=200),
    "m512_no_outliers": L3.scaled(m=512, m_out=0, n_out=0, N=500),
    "first_token": L3.scaled(N=1),
    "tile_start": L3.scaled(N=33),                             # new token opens code tile 1
    "tile_end": L3.scaled(N=32),                               # new token closes code tile 0
    "fp32_separate_calls": W["tiny_fp32"].scaled(B=2, Hq=2, Hkv=1, N=300, vmode="codes"),
    "four_bit_values": L3.scaled(nbits=4, N=700),
    "four_bit_values_70b": W["llama31_70b_gqa_decode"].scaled(B=1, Hq=16, Hkv=2, N=450, nbits=4),
    "three_bit_values": L3.scaled(nbits=3, N=701),
    "three_bit_values_70b": W["llama31_70b_gqa_decode"].scaled(B=1, Hq=16, Hkv=2, N=430, nbits=3),
    "three_bit_tile_start": L3.scaled(nbits=3, N=65),
}
BITS_SENTINEL = np.uint32(0xA5A5A5A5)
HALF_SENTINEL = np.uint16(0x3C00)     # 1.0


def dev_cache(w, kq, vq, n_prefix: int, Ncap: int):
    """Device cache of capacity Ncap: oracle rows 0 .. n_prefix-1, sentinels elsewhere."""
    Wd = (w.m + w.m_out) // 32
    bits = np.full((w.B, w.Hkv, Ncap, Wd), BITS_SENTINEL, dtype=np.uint32)
    bits[:, :, :n_prefix] = kq["bits"][:, :, :n_prefix]
    norms = np.full((w.B, w.Hkv, Ncap, 2), HALF_SENTINEL, dtype=np.uint16)
    norms[:, :, :n_prefix] = kq["norms"][:, :, :n_prefix].view(np.uint16)
    codes = np.full((w.B, w.Hkv, Ncap, w.d), 2 ** w.nbits - 1, dtype=np.uint8)
    if n_prefix:
        codes[:, :, :n_prefix] = oracle.unpack_codes(vq["codes"][:, :, :n_prefix], w.nbits, w.d)
    meta = np.full((w.B, w.Hkv, Ncap, 2), HALF_SENTINEL, dtype=np.uint16)
    meta[:, :, :n_prefix] = vq["meta"][:, :, :n_prefix].view(np.uint16)
    tiles = layout.tiles_from_codes(codes, w.nbits, Ncap)
    return qjl.Cache(bits=bits_dev(bits, w.m, w.m_out),
                     norms=torch.from_numpy(norms.view(np.float16)).cuda(),
                     codes=torch.from_numpy(tiles.view(np.int32)).cuda(),
                     meta=torch.from_numpy(meta.view(np.float16)).cuda(),
                     m=w.m, m_out=w.m_out, nbits=w.nbits)


def check_row(w, cache, kq, vq, pos: int, Ncap: int, what: str):
    """Position pos against the oracle; positions past pos keep their sentinels."""
    gb = bits_np(cache.bits, w.m, w.m_out)
    ref = {"bits": kq["bits"][:, :, pos:pos + 1], "near_zero": kq["near_zero"][:, :, pos:pos + 1]}
    nmis, _ = compare_bits(gb[:, :, pos:pos + 1], ref, f"{what} appended bits", w.m + w.m_out)
    gn = cache.norms.cpu().numpy()
    compare_norms(gn[:, :, pos:pos + 1], kq["norms"][:, :, pos:pos + 1], f"{what} appended norms")
    gc = layout.codes_from_tiles(cache.codes.cpu().numpy(), w.nbits, Ncap)
    np.testing.assert_array_equal(gc[:, :, pos], oracle.unpack_codes(vq["codes"][:, :, pos:pos + 1], w.nbits, w.d)[:, :, 0])
    gm = cache.meta.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(gm[:, :, pos], vq["meta"][:, :, pos].view(np.uint16))
    # untouched: the rest of the capacity and the prefix
    assert np.all(gb[:, :, pos + 1:] == BITS_SENTINEL)
    assert np.all(gn.view(np.uint16)[:, :, pos + 1:] == HALF_SENTINEL)
    assert np.all(gc[:, :, pos + 1:] == 2 ** w.nbits - 1)
    assert np.all(gm[:, :, pos + 1:] == HALF_SENTINEL)
    if pos:   # the prefix: the oracle's rows, or rows an earlier step appended (near-zero bits may differ)
        compare_bits(gb[:, :, :pos], {"bits": kq["bits"][:, :, :pos], "near_zero": kq["near_zero"][:, :, :pos]},
                     f"{what} prefix", w.m + w.m_out)
    if pos:
        np.testing.assert_array_equal(gc[:, :, :pos], oracle.unpack_codes(vq["codes"][:, :, :pos], w.nbits, w.d))
    same = nmis == 0 and np.array_equal(gn.view(np.uint16)[:, :, pos], kq["norms"][:, :, pos].view(np.uint16))
    return same


def run_step(w, x, cache, N, *, nsplit=0, scores=None, ws=None, estimator=0, path=0):
    B = w.B
    Kd, Vd = to_dev(x["K"], w.dtype), to_dev(x["V"], w.dtype)
    out = torch.full((B, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
    qjl.decode_step(to_dev(x["Q"], w.dtype), Kd[:, N - 1:N], Vd[:, N - 1:N], to_dev(x["S_in"], w.dtype),
                    to_dev(x["S_out"], w.dtype) if w.m_out else None,
                    torch.from_numpy(x["oidx"]).cuda() if w.n_out else None, cache, N, out,
                    scores_dbg=scores, nsplit=nsplit, workspace=ws, estimator=estimator, path=path)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_parity(name):
    w = CASES[name]
    N = w.N
    Ncap = N + 37
    log(f"[decode_step] {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={N} Ncap={Ncap} m={w.m} m_out={w.m_out} {w.dtype}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    vq = oracle.quantize_values(x["V"], w.nbits)
    cache = dev_cache(w, kq, vq, N - 1, Ncap)
    scores = torch.full((w.B, w.Hq, N), float("nan"), dtype=torch.float32, device="cuda")
    out = run_step(w, x, cache, N, scores=scores)
    same = check_row(w, cache, kq, vq, N - 1, Ncap, name)

    # the three separate calls on a copy of the same prefix write the same row and give the same output
    c2 = dev_cache(w, kq, vq, N - 1, Ncap)
    Kd, Vd = to_dev(x["K"], w.dtype), to_dev(x["V"], w.dtype)
    S_in, S_out = to_dev(x["S_in"], w.dtype), to_dev(x["S_out"], w.dtype) if w.m_out else None
    oidx = torch.from_numpy(x["oidx"]).cuda() if w.n_out else None
    qjl.quantize_keys(Kd[:, N - 1:N], S_in, S_out, oidx, c2.bits, c2.norms, t0=N - 1)
    qjl.quantize_values(Vd[:, N - 1:N], w.nbits, c2.codes, c2.meta, t0=N - 1)
    out2 = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    s2 = torch.full((w.B, w.Hq, N), float("nan"), dtype=torch.float32, device="cuda")
    qjl.decode_attention(to_dev(x["Q"], w.dtype), S_in, S_out, oidx, c2.bits, c2.norms, N, out2, codes=c2.codes,
                         meta=c2.meta, nbits=w.nbits, scores_dbg=s2)
    torch.cuda.synchronize()
    for f in ("norms", "codes", "meta"):
        np.testing.assert_array_equal(getattr(cache, f).cpu().numpy(), getattr(c2, f).cpu().numpy(), err_msg=f)
    gb, gb2 = bits_np(cache.bits, w.m, w.m_out), bits_np(c2.bits, w.m, w.m_out)
    compare_bits(gb2[:, :, N - 1:N], {"bits": gb[:, :, N - 1:N], "near_zero": kq["near_zero"][:, :, N - 1:N]},
                 f"{name} fused vs separate", w.m + w.m_out)
    if np.array_equal(gb, gb2):
        d_out = float(np.abs(out - out2.cpu().numpy()).max())
        d_sc = float(np.nanmax(np.abs(scores.cpu().numpy() - s2.cpu().numpy())))
        log(f"  {name}: fused vs separate: out {d_out:.2e}, scores {d_sc:.2e}")
        assert d_out <= 1e-5 and d_sc <= 1e-5 * max(1.0, float(np.abs(s2.cpu().numpy()).max()))

    # output against the oracle over all N positions, on the cache the GPU wrote
    log(f"  {name}: appended row {'equals' if same else 'differs in near-zero bits / a norm ulp from'} the oracle's")
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], device_cache_np(cache, w, N), N, out,
                 scores.cpu().numpy(), units, what=f"{name} step output")


@pytest.mark.parametrize("name", ["llama2_mha", "llama3_gqa", "llama31_70b_gqa", "group16", "fp32_separate_calls"])
def test_decode_step_two_sided(name):
    """The two-sided estimator through the decode step: the fused prologue takes the query signs and
    part norms (bf16), the separate calls the fp32 projection; the appended row is unchanged."""
    w = CASES[name]
    N = w.N
    Ncap = N + 5
    log(f"[decode_step two-sided] {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={N} {w.dtype}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    vq = oracle.quantize_values(x["V"], w.nbits)
    cache = dev_cache(w, kq, vq, N - 1, Ncap)
    scores = torch.full((w.B, w.Hq, N), float("nan"), dtype=torch.float32, device="cuda")
    out = run_step(w, x, cache, N, scores=scores, estimator=qjl.QJL_EST_TWO_SIDED)
    check_row(w, cache, kq, vq, N - 1, Ncap, f"{name} two-sided")
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], device_cache_np(cache, w, N), N, out,
                 scores.cpu().numpy(), units, what=f"{name} two-sided step", estimator="two_sided")


@pytest.mark.parametrize("nsplit", [1, 7])
def test_decode_step_split_counts(nsplit):
    """Forced chunk counts: one chunk (the only workgroup merges) and seven (ragged last chunk)."""
    w = CASES["llama3_gqa"]
    N, Ncap = w.N, w.N
    log(f"[decode_step] nsplit={nsplit} N={N}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    vq = oracle.quantize_values(x["V"], w.nbits)
    cache = dev_cache(w, kq, vq, N - 1, Ncap)
    out = run_step(w, x, cache, N, nsplit=nsplit)
    check_row(w, cache, kq, vq, N - 1, Ncap, f"nsplit={nsplit}")
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], device_cache_np(cache, w, N), N, out, None, units,
                 what=f"nsplit={nsplit}")


@pytest.mark.parametrize("name,N,nsplit", [
    # chunks are multiples of 512 tokens
    ("llama31_70b_gqa", 513, 2),    # the new token is the only token of chunk 1
    ("llama31_70b_gqa", 1024, 2),   # the new token closes chunk 1
    ("llama3_gqa", 1025, 3),        # the new token is the only token of chunk 2
    ("llama3_gqa", 1024, 3),        # the new token closes chunk 1, chunk 2 is empty
])
def test_decode_step_new_token_at_chunk_edges(name, N, nsplit):
    """The decode kernel's own append: the workgroup whose chunk holds position N - 1 appends the new
    token before it reads the cache; the token at either end of a chunk, alone in one, or next to an
    empty chunk gives the oracle's row and output."""
    w = CASES[name].scaled(N=N)
    Ncap = N + 3
    log(f"[decode_step chunk edge] {name} N={N} nsplit={nsplit}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    vq = oracle.quantize_values(x["V"], w.nbits)
    cache = dev_cache(w, kq, vq, N - 1, Ncap)
    scores = torch.full((w.B, w.Hq, N), float("nan"), dtype=torch.float32, device="cuda")
    out = run_step(w, x, cache, N, scores=scores, nsplit=nsplit)
    check_row(w, cache, kq, vq, N - 1, Ncap, f"{name} N={N} nsplit={nsplit}")
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], device_cache_np(cache, w, N), N, out,
                 scores.cpu().numpy(), units, what=f"{name} N={N} nsplit={nsplit}")


def test_decode_step_consecutive_steps_share_workspace():
    """Three steps in a row (N, N+1, N+2) with one workspace: nothing in the workspace carries over
    from one step to the next (every step rewrites the query operands and the chunk partials it
    reads)."""
    w = CASES["llama31_70b_gqa"].scaled(N=700)
    N0 = w.N - 2
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    vq = oracle.quantize_values(x["V"], w.nbits)
    cache = dev_cache(w, kq, vq, N0 - 1, w.N)
    ws = torch.empty(qjl.decode_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.m, w.m_out, 5), dtype=torch.uint8, device="cuda")
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    for N in (N0, N0 + 1, N0 + 2):
        log(f"[decode_step] consecutive N={N}")
        # a fixed chunk count, so that the one workspace (sized for it) serves every N
        out = run_step(w, x, cache, N, nsplit=5, ws=ws)
        check_row(w, cache, kq, vq, N - 1, w.N, f"step N={N}")
        check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], device_cache_np(cache, w, N), N, out, None, units,
                     what=f"consecutive N={N}")


def test_decode_step_rejects_bad_arguments():
    w = CASES["llama3_gqa"]
    x = inputs(w.scaled(N=64))
    cache = qjl.alloc_cache(w.B, w.Hkv, 64, w.m, w.m_out, w.nbits)
    Q = to_dev(x["Q"], w.dtype)
    Kd, Vd = to_dev(x["K"], w.dtype), to_dev(x["V"], w.dtype)
    S_in, S_out = to_dev(x["S_in"], w.dtype), to_dev(x["S_out"], w.dtype)
    oidx = torch.from_numpy(x["oidx"]).cuda()
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    with pytest.raises(qjl.QJLError) as e:
        qjl.decode_step(Q, Kd[:, :1], Vd[:, :1], S_in, S_out, oidx, cache, 65, out)     # N > Ncap
    assert e.value.status == qjl.QJL_ERR_INVALID_ARG
    with pytest.raises(qjl.QJLError) as e:
        qjl.decode_step(Q, Kd[:, :1], Vd[:, :1], S_in, S_out, oidx, cache, 0, out)      # nothing to append to
    assert e.value.status == qjl.QJL_ERR_INVALID_ARG
    # 3-bit codes decode on the matrix-core sketch shapes only (m + m_out <= 512)
    c3 = qjl.alloc_cache(w.B, w.Hkv, 64, 512, 512, 3)
    S5 = torch.zeros((512, w.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qjl.QJLError) as e:
        qjl.decode_step(Q, Kd[:, :1], Vd[:, :1], S5, S5, oidx, c3, 10, out)
    assert e.value.status == qjl.QJL_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["llama2_mha", "llama31_70b_gqa"])
def test_decode_step_vector_path(name):
    """The decode step with the vector-unit decode (the append as separate launches): the same cache
    rows, and the output against the oracle on the GPU-written cache."""
    w = CASES[name]
    N, Ncap = w.N, w.N + 3
    log(f"[decode_step vector path] {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={N}")
    x = inputs(w)
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    vq = oracle.quantize_values(x["V"], w.nbits)
    cache = dev_cache(w, kq, vq, N - 1, Ncap)
    scores = torch.full((w.B, w.Hq, N), float("nan"), dtype=torch.float32, device="cuda")
    out = run_step(w, x, cache, N, scores=scores, path=qjl.QJL_PATH_VECTOR)
    check_row(w, cache, kq, vq, N - 1, Ncap, f"{name} vector path")
    units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], device_cache_np(cache, w, N), N, out,
                 scores.cpu().numpy(), units, what=f"{name} vector-path step")
