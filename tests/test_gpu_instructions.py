"""The gfx950 instruction forms the kernels rely on, checked on the GPU against exact host models.

The decode kernels feed the query to v_mfma_scale_f32_16x16x128_f8f6f4 as fp6 e2m3 pieces with a
scale byte per lane (selected by op_sel), build those pieces with the packed fp6 conversions, and stage
block data through buffer loads with an LDS destination. These tests run each form in a small kernel
(tests/probes/qjl_probes.hip) and compare every output with a model of the operand layout and the
number formats written here; read-only kernels measure the HBM read rates the decode is compared with
(a plain streaming read, and the decode's own access pattern through its load path).
"""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libqjl_probes.so")


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(LIB_PATH), "tests/probes/libqjl_probes.so is not built (run __graft_entry__.build())"
    lib = ctypes.CDLL(LIB_PATH)
    for name in ("probe_mfma_f6f4", "probe_cvt_fp6", "probe_lds_dma", "probe_permlane_swaps", "probe_stream_read",
                 "probe_decode_stream", "probe_mfma_rate", "probe_f8f6f4_rate", "probe_fp8_pieces", "probe_lds_rate"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def e2m3(c: int) -> float:
    """fp6 e2m3: sign bit 5, exponent bits 4..3 (bias 1), mantissa bits 2..0; exponent 0 = subnormal."""
    s, e, m = (c >> 5) & 1, (c >> 3) & 3, c & 7
    v = (1.0 + m / 8.0) * 2.0 ** (e - 1) if e else m / 8.0
    return -v if s else v


def e2m1(c: int) -> float:
    """fp4 e2m1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    v = (1.0 + m / 2.0) * 2.0 ** (e - 1) if e else m / 2.0
    return -v if s else v


E2M3 = np.array([e2m3(c) for c in range(64)])


def pack_bits(values, width: int, words: int) -> np.ndarray:
    """values[i] at bits width*i of a little-endian run of 32-bit words."""
    out = np.zeros(words, dtype=np.uint64)
    for i, v in enumerate(values):
        bit = width * i
        out[bit // 32] |= (int(v) << (bit % 32)) & 0xFFFFFFFF
        if bit % 32 + width > 32:
            out[bit // 32 + 1] |= int(v) >> (32 - bit % 32)
    return out.astype(np.uint32)


def unpack_bits(words, width: int, count: int) -> list:
    w = 0
    for i, x in enumerate(words):
        w |= int(x) << (32 * i)
    return [(w >> (width * i)) & ((1 << width) - 1) for i in range(count)]


@pytest.mark.parametrize("opsel", [0, 1, 2, 3])
def test_fp6_times_fp4_operands_and_lane_scales(lib, opsel):
    """A (16 x 128, fp6) row r, K slice g is supplied by lane 16 g + r as 32 values packed from bit 0,
    scaled by byte opsel of that lane's scale word; B (128 x 16, fp4) column c, K slice g by lane 16 g + c;
    lane l receives D rows 4 (l / 16) .. + 3 of column l % 16."""
    rng = np.random.default_rng(40 + opsel)
    A = rng.integers(0, 64, (16, 128))
    Bm = rng.integers(0, 16, (128, 16))
    exps = rng.integers(0, 3, (64, 4))            # scale exponents 0..2: every partial sum exact in fp32
    a = np.zeros((64, 8), np.uint32)
    b = np.zeros((64, 8), np.uint32)
    sc = np.zeros(64, np.uint32)
    for l in range(64):
        g, r = l // 16, l % 16
        a[l, :6] = pack_bits(A[r, 32 * g: 32 * g + 32], 6, 6)
        b[l, :4] = pack_bits(Bm[32 * g: 32 * g + 32, r], 4, 4)
        sc[l] = sum(int(127 + exps[l, q]) << (8 * q) for q in range(4))
    Av = np.vectorize(e2m3)(A)
    Bv = np.vectorize(e2m1)(Bm)
    scale = np.zeros((16, 128))
    for k in range(128):
        for r in range(16):
            scale[r, k] = 2.0 ** exps[16 * (k // 32) + r, opsel]
    D = (Av * scale) @ Bv
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int32)).cuda()  # noqa: E731
    d = torch.empty(256, dtype=torch.float32, device="cuda")
    assert lib.probe_mfma_f6f4(_p(dev(a)), _p(dev(b)), _p(dev(sc)), opsel, _p(d), _stream()) == 0
    torch.cuda.synchronize()
    got = d.cpu().numpy().reshape(64, 4)
    want = np.array([[D[4 * (l // 16) + i, l % 16] for i in range(4)] for l in range(64)])
    np.testing.assert_array_equal(got, want.astype(np.float32))


def _e2m3_nearest_even(v: float) -> int:
    """The e2m3 code nearest to v, ties to the even code, magnitudes beyond 7.5 saturated."""
    if abs(v) >= 7.5:
        return 31 | (32 if v < 0 else 0)
    best, err = 0, np.inf
    for c in range(32):
        e = abs(E2M3[c] - abs(v))
        if e < err or (e == err and c % 2 == 0):
            best, err = c, e
    return best | (32 if (v < 0 and best) else 0)


def test_packed_fp6_conversions(lib):
    """v_cvt_scalef32_2xpk16_fp6_f32 rounds x / scale to the nearest e2m3 value (ties to even, saturating)
    and places element i of its first source at position 2 i, of the second at 2 i + 1;
    v_cvt_scalef32_pk32_f32_fp6 returns position j's value times scale."""
    rng = np.random.default_rng(7)
    x = np.zeros((64, 32), np.float32)
    scale = np.zeros(64, np.float32)
    for l in range(64):
        scale[l] = np.float32(2.0 ** int(rng.integers(-20, 21)))
        kind = rng.integers(0, 4, 32)
        u = np.where(kind == 0, rng.uniform(0, 7.5, 32),
                     np.where(kind == 1, rng.integers(1, 121, 32) / 16.0,          # many exact ties
                              np.where(kind == 2, rng.uniform(0.01, 1.0, 32), rng.uniform(7.5, 9.5, 32))))
        x[l] = (u * np.where(rng.random(32) < 0.5, -1, 1) * scale[l]).astype(np.float32)
    packed = torch.empty(64 * 6, dtype=torch.int32, device="cuda")
    back = torch.empty(64 * 32, dtype=torch.float32, device="cuda")
    assert lib.probe_cvt_fp6(_p(torch.from_numpy(x.ravel()).cuda()), _p(torch.from_numpy(scale).cuda()), _p(packed),
                             _p(back), _stream()) == 0
    torch.cuda.synchronize()
    pk = packed.cpu().numpy().view(np.uint32).reshape(64, 6)
    bk = back.cpu().numpy().reshape(64, 32)
    for l in range(64):
        codes = unpack_bits(pk[l], 6, 32)
        src = [x[l, j // 2] if j % 2 == 0 else x[l, 16 + j // 2] for j in range(32)]
        want = [_e2m3_nearest_even(float(v) / float(scale[l])) for v in src]
        zero = lambda c: 0 if c == 32 else c  # noqa: E731  (either sign of zero)
        assert [zero(c) for c in codes] == [zero(c) for c in want], f"lane {l}: {codes} != {want}"
        np.testing.assert_array_equal(bk[l], np.array([E2M3[c] * scale[l] for c in codes], np.float32))


def _e4m3_bits(x: np.ndarray) -> np.ndarray:
    """fp8 e4m3 (sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 subnormal, step
    2^-9) of float32 values with |x| <= 448, rounded to nearest, ties to even."""
    a = np.abs(x.astype(np.float64))
    _, ex = np.frexp(a)                          # a in [2^(ex-1), 2^ex)
    e = np.maximum(ex - 1, -6)
    q = np.round(a / np.exp2(e - 3.0))           # exact quotient; numpy rounds half to even
    carry = q >= 16
    e, q = np.where(carry, e + 1, e), np.where(carry, 8, q)
    normal = q >= 8
    field = np.where(normal, e + 7, 0).astype(np.uint32)
    mant = np.where(normal, q - 8, q).astype(np.uint32)
    return (np.signbit(x).astype(np.uint32) << 7) | (field << 3) | mant


def test_fp8_pieces_scaled_conversions(lib):
    """The three e4m3 pieces of the decode's softmax weights come from gfx950's scaled conversions (the
    scale's power of two divides before rounding and multiplies after decoding).  On 4M values (uniform
    weights in [0, 256), magnitudes from 2^-12 to 2^8 of either sign, exact e4m3 ties) they equal the
    pieces of the unscaled conversions of v, 16 r1 and 256 r2, bit for bit, and the first piece is
    e4m3(v) rounded to nearest even by the host model."""
    rng = np.random.default_rng(21)
    n = 1 << 22
    kind = rng.integers(0, 3, n)
    uni = rng.uniform(0.0, 256.0, n)
    wide = np.exp2(rng.uniform(-12.0, 8.0, n)) * np.where(rng.random(n) < 0.5, -1.0, 1.0)
    tie = (rng.integers(8, 16, n) + 0.5) * np.exp2(rng.integers(-6, 8, n) - 3.0)
    x = np.where(kind == 0, uni, np.where(kind == 1, wide, tie)).astype(np.float32)
    x[x == 0] = np.float32(1.0)
    xd = torch.from_numpy(x).cuda()
    scaled = torch.empty(3 * n // 4, dtype=torch.int32, device="cuda")
    plain = torch.empty(3 * n // 4, dtype=torch.int32, device="cuda")
    assert lib.probe_fp8_pieces(_p(xd), n // 4, _p(scaled), _p(plain), _stream()) == 0
    torch.cuda.synchronize()
    sw = scaled.cpu().numpy().view(np.uint32).reshape(-1, 3)
    pw = plain.cpu().numpy().view(np.uint32).reshape(-1, 3)
    first = np.stack([(sw[:, 0] >> (8 * j)) & 0xFF for j in range(4)], axis=1).ravel()
    np.testing.assert_array_equal(first, _e4m3_bits(x))
    np.testing.assert_array_equal(sw, pw)


def test_lds_read_rate_of_the_key_fragments(lib):
    """64-lane 16-byte LDS reads in the key quantizer's A-fragment pattern (lane l: row l % 32, bytes
    16 (l / 32) + 32 s of its row), 16 waves per workgroup: with the kernel's 272-byte row pitch the 32
    rows of a read fall on distinct banks and it runs at the full LDS rate; with 256-byte rows every
    lane of a half-wave hits the same banks.  Bytes per shader clock per CU (`pytest -s` prints them)."""
    iters, blocks = 2000, 256
    rate = {}
    for pitch in (272, 256):
        clocks = torch.zeros(blocks, dtype=torch.int64, device="cuda")
        sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
        for _ in range(2):                       # the second launch is timed
            assert lib.probe_lds_rate(iters, pitch, blocks, _p(clocks), _p(sink), _stream()) == 0
        torch.cuda.synchronize()
        rate[pitch] = 16 * iters * 8 * 1024 / float(np.median(clocks.cpu().numpy()))
    print(f"LDS read rate, bytes per clock per CU: {rate[272]:.0f} with 272-byte rows, {rate[256]:.0f} with 256-byte rows")
    assert rate[272] >= 4.0 * rate[256]          # measured 237 against 16
    assert rate[272] >= 160.0


@pytest.mark.parametrize("size", [4, 16])
def test_lds_destination_loads(lib, size):
    """A buffer load with an LDS destination writes lane l's `size` bytes at LDS offset size * l
    (after M0), whatever global offset the lane reads."""
    rng = np.random.default_rng(size)
    src = rng.integers(0, 2**32, 256, dtype=np.uint64).astype(np.uint32)
    off = (rng.permutation(1024 // size)[:64] * size).astype(np.int32)
    out = torch.empty(64 * size // 4, dtype=torch.int32, device="cuda")
    assert lib.probe_lds_dma(_p(torch.from_numpy(src.view(np.int32)).cuda()), _p(torch.from_numpy(off).cuda()), size,
                             _p(out), _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    want = np.concatenate([src[o // 4: o // 4 + size // 4] for o in off])
    np.testing.assert_array_equal(got, want)


def test_permlane_swaps(lib):
    """v_permlane16_swap(a, b) exchanges the odd 16-lane rows of a with the even rows of b (row r + 1 of
    a <-> row r of b); v_permlane32_swap(a, b) the upper 32 lanes of a with the lower 32 of b.  The
    four-wave decode transposes its code pieces across lane rows with these two."""
    rng = np.random.default_rng(3)
    a = rng.integers(0, 2**32, 64, dtype=np.uint64).astype(np.uint32)
    b = rng.integers(0, 2**32, 64, dtype=np.uint64).astype(np.uint32)
    out = torch.empty(256, dtype=torch.int32, device="cuda")
    dev = lambda x: torch.from_numpy(x.view(np.int32)).cuda()  # noqa: E731
    assert lib.probe_permlane_swaps(_p(dev(a)), _p(dev(b)), _p(out), _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).reshape(4, 64)
    a16, b16, a32, b32 = a.copy(), b.copy(), a.copy(), b.copy()
    for l in range(64):
        if (l // 16) % 2 == 1:
            a16[l] = b[l - 16]
        else:
            b16[l] = a[l + 16]
        if l >= 32:
            a32[l] = b[l - 32]
        else:
            b32[l] = a[l + 32]
    np.testing.assert_array_equal(got, np.stack([a16, b16, a32, b32]))


def _rate(launch, nbytes: int, reps: int = 10) -> float:
    for _ in range(2):
        assert launch() == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    return nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9


@pytest.mark.parametrize("blocks", [2048, 8192])
def test_stream_read_rate(lib, blocks):
    """The HBM read rate of a plain 16-byte streaming read, with ordinary and with non-temporal loads,
    printed (the practical ceiling for a memory-bound kernel on this GPU); asserted only to be a sane
    fraction of the 8 TB/s peak."""
    n16 = (2 << 30) // 16
    buf = torch.ones(n16 * 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    for nt in (0, 1):
        gbs = _rate(lambda: lib.probe_stream_read(_p(buf), ctypes.c_int64(n16), _p(sink), blocks, nt, _stream()), n16 * 16)
        kind = "non-temporal" if nt else "plain"
        print(f"\n[stream read] 2 GiB, {blocks} workgroups x 256, {kind}: {gbs:.0f} GB/s ({gbs / 8000 * 100:.1f}% of 8 TB/s)")
        assert gbs > 3000


def test_decode_stream_rates(lib):
    """The cache-read pattern of the eight-wave decode on its Llama-3.1-70B shape (128 (sequence, KV head)
    units of 131072 tokens, two chunks each, 104 B per token: 1.745 GB), with no arithmetic: through the
    decode's LDS-destination loads (whole code tiles per load: the decode's own load path), the same with
    the code words loaded as 16-byte pieces 64 bytes apart (the layout it replaced), and into registers.
    Printed; asserted only to be a sane fraction of the 8 TB/s peak."""
    U, Ncap, ns = 128, 131072, 2
    sg = torch.ones(U * Ncap * 16, dtype=torch.int32, device="cuda")
    nr = torch.ones(U * Ncap, dtype=torch.int32, device="cuda")
    mt = torch.ones(U * Ncap, dtype=torch.int32, device="cuda")
    cd = torch.ones(U * Ncap * 8, dtype=torch.int32, device="cuda")
    blocks = (U * ns + 7) // 8 * 8
    sink = torch.empty(blocks * 512, dtype=torch.int32, device="cuda")
    nbytes = U * Ncap * 104
    kinds = {1: "LDS-destination loads, whole code tiles", 2: "LDS-destination loads, strided code pieces",
             0: "register loads"}
    for mode, kind in kinds.items():
        gbs = _rate(lambda: lib.probe_decode_stream(_p(sg), _p(nr), _p(mt), _p(cd), ctypes.c_int64(Ncap), U, ns, mode,
                                                    _p(sink), _stream()), nbytes)
        print(f"\n[decode stream] 1.745 GB, {blocks} workgroups x 512, {kind}: {gbs:.0f} GB/s "
              f"({gbs / 8000 * 100:.1f}% of 8 TB/s, {nbytes / gbs / 1e3:.1f} us)")
        assert gbs > 3000


def test_bf16_matrix_core_rate(lib):
    """The rate of v_mfma_f32_32x32x16_bf16 with register operands only (four independent accumulator
    chains per wave; 2, 4 and 8 waves per SIMD): the practical ceiling of a bf16 contraction such as the
    key quantizer's, printed against the 2.5 PFLOP/s dense figure; asserted only to be sane."""
    rng = np.random.default_rng(11)
    vals = (rng.standard_normal(128 * 8) * 1e-2).astype(np.float32)
    src = torch.from_numpy(vals).cuda().to(torch.bfloat16)
    iters = 4096
    best = 0.0
    for blocks in (512, 1024, 2048):
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        flops = blocks * 4 * iters * 4 * 2.0 * 32 * 32 * 16
        tfs = _rate(lambda: lib.probe_mfma_rate(_p(src), iters, blocks, _p(out), _stream()), flops) / 1e3
        print(f"\n[matrix cores] v_mfma_f32_32x32x16_bf16, register operands, {blocks * 4 // 1024} waves per SIMD: "
              f"{tfs:.0f} TFLOP/s ({tfs / 2500 * 100:.1f}% of 2.5 PFLOP/s)")
        assert torch.isfinite(out).all()
        best = max(best, tfs)
    assert best > 300


def test_fp6_and_fp8_query_operand_issue_rates(lib):
    """v_mfma_scale_f32_16x16x128_f8f6f4 with B in fp4, A in fp6 e2m3 (the decode's score operand) or in
    fp8 e4m3 (its value operand), register operands only, four independent chains per wave, 8 waves
    per SIMD: printed as TFLOP/s and the fp8 / fp6 time ratio; asserted only that fp6 is not slower."""
    rng = np.random.default_rng(12)
    src = torch.from_numpy(rng.integers(0, 2**32, 1024, dtype=np.uint64).astype(np.uint32).view(np.int32)).cuda()
    blocks, iters = 2048, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    flops = blocks * 4 * iters * 4 * 2.0 * 16 * 16 * 128
    rates = {}
    for fp6, name in ((1, "fp6 x fp4"), (0, "fp8 x fp4")):
        rates[name] = _rate(lambda: lib.probe_f8f6f4_rate(_p(src), fp6, iters, blocks, _p(out), _stream()), flops) / 1e3
        print(f"\n[matrix cores] v_mfma_scale_f32_16x16x128_f8f6f4, {name}: {rates[name]:.0f} TFLOP/s")
    print(f"\n[matrix cores] fp8 x fp4 takes {rates['fp6 x fp4'] / rates['fp8 x fp4']:.2f}x the time of fp6 x fp4")
    assert rates["fp6 x fp4"] >= 0.95 * rates["fp8 x fp4"]
