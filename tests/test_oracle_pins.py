"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test ties an oracle function to something other than itself: a worked example printed on a page
(fixtures under tests/golden/, each citing its page and section), a closed form, an invariant, a
special case that reduces to a textbook routine, or a brute-force search on a tiny input.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ page 5: uniform 2-bit quantizer

def test_uniform_quantizer_single_value_and_centroids():
    g = golden("page5_uniform_2bit.json")
    sv = g["single_value_printed"]
    idx, rec = oracle.uniform_quantize(sv["x"])
    assert int(idx) == sv["bucket"]
    assert float(rec) == pytest.approx(sv["reconstructed"], abs=1e-12)
    assert abs(sv["x"] - float(rec)) == pytest.approx(sv["error"], abs=1e-12)
    # bucket midpoints of [-1, 1] in 4 equal buckets; the right edge 1.0 belongs to the last bucket
    _, centroids = oracle.uniform_quantize(np.array([-0.9, -0.3, 0.2, 0.9, 1.0, -1.0]))
    assert list(centroids) == [-0.75, -0.25, 0.25, 0.75, 0.75, -0.75]
    assert list(centroids[:4]) == g["bucket_centroids_printed"]


def test_uniform_quantizer_worked_example_and_page_errors():
    g = golden("page5_uniform_2bit.json")
    k, q = np.array(g["k"]), np.array(g["q"])
    assert float(q @ k) == pytest.approx(g["true_dot_printed"], abs=5e-5)
    idx, rec = oracle.uniform_quantize(k)
    # by the page's own bucket edges 0.41 lies in [0, 0.5) -> bucket 2 (the page prints 3)
    assert list(idx) == [2, 2, 1, 3, 1, 3, 2, 1]
    assert list(idx) != g["bucket_row_printed"]
    assert float(q @ rec) == pytest.approx(-0.7925, abs=1e-12)
    # the page's printed bucket row gives -0.9025, not the printed -0.6150
    printed_rec = -0.75 + 0.5 * np.array(g["bucket_row_printed"])
    assert float(q @ printed_rec) == pytest.approx(-0.9025, abs=1e-12)
    # -0.6150 is reached by no assignment of the 8 coordinates to the 4 centroids (brute force)
    cents = np.array([-0.75, -0.25, 0.25, 0.75])
    reach = {round(float(q @ cents[list(a)]), 4) for a in itertools.product(range(4), repeat=8)}
    assert round(g["quantized_dot_printed"], 4) not in reach
    assert round(-0.7925, 4) in reach and round(-0.9025, 4) in reach


# ------------------------------------------------------------------ page 3: token-wise min/max values

def test_tokenwise_two_bit_page_example():
    g = golden("page3_tokenwise.json")["two_bit"]
    v = np.array([g["v"]], dtype=np.float32)
    codes, meta = oracle.quantize_value_vectors(v, 2)
    assert list(codes[0]) == g["codes_printed"]
    mn, step = float(meta[0, 0]), float(meta[0, 1])
    levels = [mn + i * step for i in range(4)]
    np.testing.assert_allclose(levels, g["levels_printed"], atol=1e-3)   # fp16 min and step
    rec = oracle.dequantize_value_vectors(codes, meta)[0]
    np.testing.assert_allclose(rec, g["reconstructed_printed"], atol=1e-3)
    qv = np.array(g["query"])
    assert float(qv @ np.array(g["v"])) == pytest.approx(g["dot_original_printed"], abs=1e-9)
    assert float(qv @ rec) == pytest.approx(g["dot_compressed_printed"], abs=2e-3)


def test_tokenwise_three_bit_outlier_page_example():
    g = golden("page3_tokenwise.json")["three_bit_outliers"]
    v = np.array([g["v"]], dtype=np.float32)
    codes, meta = oracle.quantize_value_vectors(v, 3)
    assert list(codes[0]) == g["codes_printed"]
    assert float(meta[0, 1]) == pytest.approx(g["step_printed"], abs=0.01)
    levels = [float(meta[0, 0]) + i * float(meta[0, 1]) for i in range(8)]
    np.testing.assert_allclose(levels, g["levels_printed"], atol=0.06)
    rec = oracle.dequantize_value_vectors(codes, meta)[0]
    np.testing.assert_allclose(rec, g["reconstructed_printed"], atol=0.06)
    qv = np.array(g["query"], dtype=np.float64)
    assert float(qv @ np.array(g["v"])) == pytest.approx(g["dot_original_printed"], abs=1e-9)
    assert float(qv @ rec) == pytest.approx(g["dot_compressed_printed"], abs=0.1)


def test_page_softmax_examples():
    g3 = golden("page3_tokenwise.json")["softmax"]
    np.testing.assert_allclose(oracle.softmax(g3["scores_original"]), g3["weights_original_printed"], atol=0.006)
    np.testing.assert_allclose(oracle.softmax(g3["scores_compressed"]), g3["weights_compressed_printed"], atol=0.01)
    g1 = golden("page1_one_bit_keys.json")
    for case in ("softmax_correct", "softmax_truncated"):
        np.testing.assert_allclose(oracle.softmax(g1[case]["scores"]), g1[case]["weights_printed"], atol=0.006)
    # closed form for two scores: the logistic function of their difference
    a, b = 12.83, 12.23
    assert oracle.softmax([a, b])[0] == pytest.approx(1.0 / (1.0 + math.exp(b - a)), rel=1e-14)


# ------------------------------------------------------------------ value quantizer properties

@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_value_quantizer_properties(nbits):
    rng = np.random.default_rng(7)
    v = si.round_bf16(rng.standard_normal((300, 128)).astype(np.float32) * 1.7)
    codes, meta = oracle.quantize_value_vectors(v, nbits)
    L = 2 ** nbits - 1
    assert codes.min() >= 0 and codes.max() <= L
    rows = np.arange(v.shape[0])
    assert np.all(codes[rows, v.argmin(axis=1)] == 0)
    assert np.all(codes[rows, v.argmax(axis=1)] == L)
    # brute-force nearest level (fp32 arithmetic on the stored fp16 min and step) equals rint
    mn = meta[:, 0].astype(np.float32)[:, None]
    step = meta[:, 1].astype(np.float32)[:, None]
    levels = np.arange(L + 1, dtype=np.float32)
    dist = np.abs((v - mn)[..., None] / step[..., None] - levels)      # distance in steps
    nearest = dist.argmin(axis=-1)
    ties = np.isclose(np.sort(dist, axis=-1)[..., 0], np.sort(dist, axis=-1)[..., 1], rtol=0, atol=1e-6)
    assert np.all((nearest == codes) | ties)
    # reconstruction error: half a step plus the fp16 rounding of the minimum
    rec = oracle.dequantize_value_vectors(codes, meta)
    slack = np.abs(v.min(axis=1) - meta[:, 0].astype(np.float64))[:, None]
    assert np.all(np.abs(v - rec) <= step.astype(np.float64) / 2 * (1 + 1e-3) + slack + 1e-6)


def test_value_quantizer_constant_vector_gives_zero_codes():
    v = np.full((2, 128), 0.625, dtype=np.float32)
    codes, meta = oracle.quantize_value_vectors(v, 2)
    assert np.all(codes == 0) and np.all(meta[:, 1] == 0)
    np.testing.assert_array_equal(oracle.dequantize_value_vectors(codes, meta), 0.625)


def test_code_packing_layout():
    # 2-bit: code c at bits 2c..2c+1 of the row's byte stream
    assert list(oracle.pack_codes(np.array([[1, 2, 3, 0]]), 2)[0]) == [0b00111001]
    # 3-bit: an LSB-first bit stream across byte boundaries
    assert list(oracle.pack_codes(np.array([[1, 2, 3, 4, 5, 6, 7, 0]]), 3)[0]) == [0xD1, 0x58, 0x1F]
    rng = np.random.default_rng(1)
    for nb in (2, 3, 4):
        c = rng.integers(0, 2 ** nb, size=(5, 128))
        np.testing.assert_array_equal(oracle.unpack_codes(oracle.pack_codes(c, nb), nb, 128), c)


# ------------------------------------------------------------------ keys: signs, packing, norms

def test_bit_packing_layout():
    for j in (0, 5, 31, 32, 63, 200):
        bits = np.zeros((1, 256), dtype=bool)
        bits[0, j] = True
        words = oracle.pack_bits(bits)[0]
        expect = np.zeros(8, dtype=np.uint32)
        expect[j // 32] = np.uint32(1) << np.uint32(j % 32)
        np.testing.assert_array_equal(words, expect)


def tiled_identity(d, m):
    return np.tile(np.eye(d), (m // d, 1))


def test_identity_projection_gives_page_sign_vector():
    g = golden("page1_one_bit_keys.json")
    k = np.array([g["keys"]["cat"]])
    r = oracle.quantize_key_vectors(k, tiled_identity(8, 32), np.zeros((0, 8)), [])
    signs = np.where(oracle.unpack_bits(r["bits"], 32)[0, :8], 1, -1)
    assert list(signs) == g["cat_sign_vector_printed"]
    assert int(r["bits"][0, 0]) == 0xD5D5D5D5      # [+,-,+,-,+,-,+,+] LSB-first, tiled 4x


def test_identity_projection_reconstructs_norm_times_signs():
    """S = I (tiled): the estimator is sqrt(pi/2)/d * <q, ||k|| sign(k)>, i.e. the page's
    'reconstructed key = norm x signs' dotted with the query, with the unbiasing constant."""
    g = golden("page1_one_bit_keys.json")
    q = np.array(g["query_on"])
    assert float(q @ np.array(g["keys"]["cat"])) == pytest.approx(g["score_on_cat_printed"], abs=2e-3)
    S = tiled_identity(8, 32)
    for name, kv in g["keys"].items():
        k = np.array([kv])
        r = oracle.quantize_key_vectors(k, S, np.zeros((0, 8)), [])
        sq_in, sq_out = oracle.project_query(q, S, np.zeros((0, 8)), [])
        s = oracle.estimator_scores(sq_in, sq_out, r["bits"], r["norms"])[0]
        norm16 = float(np.float16(np.linalg.norm(kv)))
        expect = math.sqrt(math.pi / 2) / 8 * norm16 * float(q @ np.sign(kv))
        assert s == pytest.approx(expect, rel=1e-13)


def test_norms_closed_form_and_fp16_rounding():
    k = np.zeros((1, 8))
    k[0, 0], k[0, 1] = 3.0, 4.0
    S = tiled_identity(8, 32)
    r = oracle.quantize_key_vectors(k, S, S, [1])
    assert r["norms"][0].tolist() == [3.0, 4.0]
    r = oracle.quantize_key_vectors(k, S, np.zeros((0, 8)), [])
    assert r["norms"][0].tolist() == [5.0, 0.0]
    # fp16 round-to-nearest-even: ties go to the even significand
    assert float(oracle.fp16(1 + 2 ** -11)) == 1.0
    assert float(oracle.fp16(1 + 3 * 2 ** -11)) == 1 + 2 ** -9
    assert float(oracle.fp16(2049.0)) == 2048.0 and float(oracle.fp16(2051.0)) == 2052.0
    rng = np.random.default_rng(3)
    kk = rng.standard_normal((50, 128)) * 3
    r = oracle.quantize_key_vectors(kk, rng.standard_normal((64, 128)), rng.standard_normal((64, 128)), [2, 9])
    mask = np.zeros(128, bool)
    mask[[2, 9]] = True
    np.testing.assert_array_equal(r["norms"][:, 0], np.linalg.norm(kk[:, ~mask], axis=1).astype(np.float16))
    np.testing.assert_array_equal(r["norms"][:, 1], np.linalg.norm(kk[:, mask], axis=1).astype(np.float16))


def test_sign_invariants():
    rng = np.random.default_rng(11)
    S_in = si.round_bf16(rng.standard_normal((256, 128)).astype(np.float32))
    S_out = si.round_bf16(rng.standard_normal((256, 128)).astype(np.float32))
    k = si.round_bf16(rng.standard_normal((64, 128)).astype(np.float32))
    ch = [3, 70, 101]
    base = oracle.quantize_key_vectors(k, S_in, S_out, ch)
    for e in (-3, 0, 5):  # exact power-of-two scaling keeps every sign
        r = oracle.quantize_key_vectors(k * 2.0 ** e, S_in, S_out, ch)
        np.testing.assert_array_equal(r["bits"], base["bits"])
    neg = oracle.quantize_key_vectors(-k, S_in, S_out, ch)
    nz = base["proj"] != 0
    b0 = oracle.unpack_bits(base["bits"], 512)
    b1 = oracle.unpack_bits(neg["bits"], 512)
    assert np.all(b1[nz] == ~b0[nz])
    # a key that is zero on every inlier channel has all inlier bits set (sign(0) = +1)
    kz = np.zeros((1, 128))
    kz[0, ch] = [1.0, -2.0, 3.0]
    rz = oracle.quantize_key_vectors(kz, S_in, S_out, ch)
    assert np.all(rz["bits"][0, :8] == 0xFFFFFFFF)
    assert rz["norms"][0, 0] == 0


def test_projection_orientation_uses_rows_of_S():
    """S is m x d and projects with its rows: a one-hot key picks column c of S."""
    rng = np.random.default_rng(5)
    S = rng.standard_normal((32, 8))
    for c in range(8):
        k = np.zeros((1, 8))
        k[0, c] = 1.0
        r = oracle.quantize_key_vectors(k, S, np.zeros((0, 8)), [])
        np.testing.assert_array_equal(oracle.unpack_bits(r["bits"], 32)[0], S[:, c] >= 0)


# ------------------------------------------------------------------ estimator closed forms and invariants

def _score(q, k, S_in, S_out, ch):
    r = oracle.quantize_key_vectors(k[None, :], S_in, S_out, ch)
    sq_in, sq_out = oracle.project_query(q, S_in, S_out, ch)
    return oracle.estimator_scores(sq_in, sq_out, r["bits"], r["norms"])[0]


def test_estimator_antisymmetric_in_q_and_positive_for_q_equal_k():
    rng = np.random.default_rng(2)
    S_in, S_out = rng.standard_normal((256, 128)), rng.standard_normal((256, 128))
    ch = [1, 50, 77, 120]
    for _ in range(5):
        q, k = rng.standard_normal(128), rng.standard_normal(128)
        assert _score(-q, k, S_in, S_out, ch) == -_score(q, k, S_in, S_out, ch)
        # q = k (no outlier split): sqrt(pi/2)/m * ||k||_16 * sum_j |(S k)_j|
        s = _score(k, k, S_in, np.zeros((0, 128)), [])
        expect = math.sqrt(math.pi / 2) / 256 * float(np.float16(np.linalg.norm(k))) * np.abs(S_in @ k).sum()
        assert s == pytest.approx(expect, rel=1e-12) and s > 0


def test_estimator_one_dimensional_closed_form():
    """d = 1: sign(s k) s q = |s| q sign(k), so score = sqrt(pi/2) q |k|_16 sign(k) mean|s|."""
    rng = np.random.default_rng(9)
    S = rng.standard_normal((64, 1))
    for q, k in ((0.7, -1.3), (-2.0, 0.25), (1.5, 3.0)):
        s = _score(np.array([q]), np.array([k]), S, np.zeros((0, 1)), [])
        expect = math.sqrt(math.pi / 2) * q * float(np.float16(abs(k))) * math.copysign(1, k) * np.abs(S).mean()
        assert s == pytest.approx(expect, rel=1e-12)


def test_outlier_split_adds_two_independent_sketches():
    """A key living only on its outlier channels is seen only by S_out, and only through the
    query's outlier channels; a query without outlier-channel mass gets no outlier term."""
    rng = np.random.default_rng(4)
    S_in, S_out = rng.standard_normal((64, 16)), rng.standard_normal((64, 16))
    ch = [2, 11]
    k = np.zeros(16)
    k[ch] = [5.0, -7.0]
    q = rng.standard_normal(16)
    s = _score(q, k, S_in, S_out, ch)
    kk = k[ch][None, :]
    sub = oracle.quantize_key_vectors(kk, S_out[:, ch], np.zeros((0, 2)), [])
    sq, _ = oracle.project_query(q[ch], S_out[:, ch], np.zeros((0, 2)), [])
    assert s == pytest.approx(oracle.estimator_scores(sq, np.zeros(0), sub["bits"], sub["norms"])[0], rel=1e-12)
    q2 = q.copy()
    q2[ch] = 0.0
    assert _score(q2, k, S_in, S_out, ch) == 0.0


# ------------------------------------------------------------------ attention closed forms and invariants

def test_attention_special_cases():
    rng = np.random.default_rng(6)
    V = rng.standard_normal((37, 16))
    np.testing.assert_allclose(oracle.attend(np.full(37, 2.5), V, 0.3), V.mean(axis=0), rtol=0, atol=1e-14)
    s = np.zeros(37)
    s[5] = 1e4
    np.testing.assert_allclose(oracle.attend(s, V, 1.0), V[5], rtol=0, atol=1e-12)
    s = rng.standard_normal(37) * 3
    perm = rng.permutation(37)
    np.testing.assert_allclose(oracle.attend(s[perm], V[perm], 0.7), oracle.attend(s, V, 0.7), atol=1e-13)
    # two keys: weight of the first is the logistic function of the scaled score gap
    o = oracle.attend(np.array([1.0, -0.5]), V[:2], 0.8)
    w = 1 / (1 + math.exp(-0.8 * 1.5))
    np.testing.assert_allclose(o, w * V[0] + (1 - w) * V[1], atol=1e-14)
    assert np.all(oracle.attend(np.zeros(0), V[:0], 1.0) == 0)


def test_memory_accounting_closed_form():
    """Bytes per token and KV head of the Llama-2-7B-shaped cache: 64 B signs + 4 B norms + 32 B
    codes + 4 B min/step = 104 B -> (m + m_out + 32 + d b + 32) / (2 d) = 3.25 bits per number,
    against the QJL summary's 3 bits per number and ~81% reduction ("Key results")."""
    w = si.WORKLOADS["llama2_7b_decode"]
    rng = np.random.default_rng(0)
    K = rng.standard_normal((1, 4, 1, 128)).astype(np.float32)
    S_in, S_out = rng.standard_normal((256, 128)), rng.standard_normal((256, 128))
    kq = oracle.quantize_keys(K, S_in, S_out, np.array([[0, 1, 2, 3]]))
    vq = oracle.quantize_values(K, 2)
    per_token = (kq["bits"].nbytes + kq["norms"].nbytes + vq["codes"].nbytes + vq["meta"].nbytes) / 4
    assert per_token == 104
    bits_per_number = per_token * 8 / (2 * w.d)
    assert bits_per_number == (w.m + w.m_out + 32 + w.d * w.nbits + 32) / (2 * w.d) == 3.25
    assert 1 - bits_per_number / 16 == pytest.approx(0.796875)
    assert 1 - 3 / 16 == pytest.approx(0.8125)


# ------------------------------------------------------------------ brute force on d = 8 inputs

def test_decode_brute_force_d8_page_vectors():
    """Whole decode on the pages' 8-dim keys, values and query, against an explicit loop over
    every projection row with +1/-1 written out (no packing, no matrices)."""
    g = golden("page1_one_bit_keys.json")
    names = ["cat", "sat", "mat"]
    K = np.array([g["keys"][n] for n in names], dtype=np.float32)
    V = np.array([g["values"][n] for n in names], dtype=np.float32)
    q = np.array(g["query_on"], dtype=np.float32)
    rng = np.random.default_rng(8)
    for m, m_out, ch in ((32, 0, []), (64, 32, [0, 3]), (256, 64, [4])):
        S_in = rng.standard_normal((m, 8))
        S_out = rng.standard_normal((m_out, 8))
        oc = np.array([ch], dtype=np.int32) if ch else np.zeros((1, 0), np.int32)
        kq = oracle.quantize_keys(K[None, :, None, :], S_in, S_out, oc)
        vq = oracle.quantize_values(V[None, :, None, :], 2)
        res = oracle.decode_attention(q[None, None, :], S_in, S_out, oc, kq["bits"], kq["norms"], 3,
                                      codes=vq["codes"], meta=vq["meta"], nbits=2, sm_scale=0.5)
        # literal evaluation
        scores = []
        for t in range(3):
            total = 0.0
            for S, sel, mm in ((S_in, [c not in ch for c in range(8)], m), (S_out, [c in ch for c in range(8)], m_out)):
                if mm == 0:
                    continue
                kt = [float(K[t, c]) if sel[c] else 0.0 for c in range(8)]
                qt = [float(q[c]) if sel[c] else 0.0 for c in range(8)]
                norm = float(np.float16(math.sqrt(sum(x * x for x in kt))))
                acc = 0.0
                for j in range(mm):
                    pk = sum(S[j, c] * kt[c] for c in range(8))
                    pq = sum(S[j, c] * qt[c] for c in range(8))
                    acc += pq * (1.0 if pk >= 0 else -1.0)
                total += math.sqrt(math.pi / 2) / mm * norm * acc
            scores.append(total)
        np.testing.assert_allclose(res["scores"][0, 0], scores, rtol=1e-12, atol=1e-12)
        vhat = []
        for t in range(3):
            vt = [float(x) for x in V[t]]
            lo, hi = min(vt), max(vt)
            step = float(np.float16(np.float32(hi - lo) / np.float32(3)))
            mn = float(np.float16(lo))
            vhat.append([mn + step * min(3, max(0, round((x - mn) / step))) for x in vt])
        z = [0.5 * s for s in scores]
        mz = max(z)
        e = [math.exp(x - mz) for x in z]
        o = [sum(e[t] * vhat[t][c] for t in range(3)) / sum(e) for c in range(8)]
        np.testing.assert_allclose(res["out"][0, 0], o, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- outlier channels

def test_select_outliers_page_examples():
    """The pages' own outlier channels: the two 100x coordinates of the 8-dim key (page 3, 'The Real
    Problem: Outlier Channels'), the four big dims of cat/sat/mat (page 1, 'Seeing It With Real
    Numbers') and the three ~0.8 dims among ~0.05 ones (page 5, 'The Third Problem: Magnitude
    Outliers')."""
    g3 = golden("page3_tokenwise.json")["three_bit_outliers"]
    K = np.array(g3["v"], dtype=np.float64).reshape(1, 1, 1, -1)
    assert oracle.select_outliers(K, 2)[0].tolist() == [c - 1 for c in g3["outlier_dims_printed_one_based"]]
    g1 = golden("page1_one_bit_keys.json")
    K = np.array([g1["keys"][t] for t in ("cat", "sat", "mat")], dtype=np.float64).reshape(1, 3, 1, -1)
    assert oracle.select_outliers(K, 4)[0].tolist() == [c - 1 for c in g1["big_dims_printed_one_based"]]
    g5 = golden("page5_uniform_2bit.json")["outlier_magnitudes_conceptual"]
    rng = np.random.default_rng(7)
    mag = np.full(g5["d"], g5["normal_magnitude"])
    mag[g5["channels"]] = g5["outlier_magnitude"]
    K = (mag * rng.choice([-1.0, 1.0], size=(2, 50, 1, g5["d"]))) * rng.uniform(0.5, 1.5, size=(2, 50, 1, g5["d"]))
    assert oracle.select_outliers(K, 3)[0].tolist() == g5["channels"]


def test_select_outliers_closed_forms_and_ties():
    d = 16
    # |k_c| = c + 1 for every key: the n_out highest channels
    K = np.tile(np.arange(1.0, d + 1.0) * np.array([1, -1] * (d // 2)), (2, 3, 2, 1))
    assert oracle.select_outliers(K, 3).tolist() == [[13, 14, 15]] * 2
    # all magnitudes equal: the lowest channels win the ties
    assert oracle.select_outliers(np.ones((1, 4, 1, d)), 5)[0].tolist() == [0, 1, 2, 3, 4]
    # the statistic is the mean of |k_c| over all 8 keys of the head (not the max, not the RMS)
    K = np.zeros((2, 4, 1, d))
    K[1, 3, 0, 7] = 1.0                                                   # mean 0.125  (max 1,   RMS 0.354)
    K[:, :, 0, 4] = 0.1                                                   # mean 0.1    (max 0.1, RMS 0.1)
    K[0, 0, 0, 9] = 0.5                                                   # mean 0.0625 (max 0.5, RMS 0.177)
    K[:, :, 0, 12] = 0.11                                                 # mean 0.11   (max 0.11, RMS 0.11)
    assert oracle.select_outliers(K, 1)[0].tolist() == [7]
    assert oracle.select_outliers(K, 2)[0].tolist() == [7, 12]           # by max or RMS: [7, 9]
    assert oracle.select_outliers(K, 3)[0].tolist() == [4, 7, 12]        # by max or RMS: [7, 9, 12]
    assert oracle.select_outliers(K, 0).shape == (1, 0)


def test_select_outliers_invariances():
    """Invariant under token order, signs, positive scale and splitting the keys into sequences;
    heads are independent."""
    rng = np.random.default_rng(3)
    K = rng.standard_normal((2, 40, 3, 32)) * rng.uniform(0.1, 3.0, size=(1, 1, 3, 32))
    ref = oracle.select_outliers(K, 5)
    assert np.array_equal(oracle.select_outliers(K[:, ::-1], 5), ref)
    assert np.array_equal(oracle.select_outliers(-2.5 * K, 5), ref)
    assert np.array_equal(oracle.select_outliers(K.reshape(1, 80, 3, 32), 5), ref)
    for h in range(3):
        assert np.array_equal(oracle.select_outliers(K[:, :, h:h + 1], 5)[0], ref[h])
    assert all(np.all(np.diff(r) > 0) for r in ref)                      # ascending, distinct


# ----------------------------------------------------------------------------- estimator variants

def test_two_sided_scores_parallel_and_antiparallel_are_exact():
    """Both sides as signs: a query parallel to the key agrees on every sign, so each part scores
    ||q_part|| * ||k_part|| (stored fp16 norm) exactly; an antiparallel query disagrees everywhere."""
    rng = np.random.default_rng(41)
    d, m, ch = 32, 64, [3, 17]
    S_in, S_out = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    k = rng.standard_normal(d)
    kq = oracle.quantize_key_vectors(k[None, :], S_in, S_out, ch)
    mask = oracle.outlier_mask(d, ch)
    n16 = kq["norms"][0].astype(np.float64)
    for c, sign in ((3.0, 1.0), (-0.5, -1.0)):
        q = c * k
        sq_in, sq_out = oracle.project_query(q, S_in, S_out, ch)
        qn_in, qn_out = np.linalg.norm(q * (1 - mask)), np.linalg.norm(q * mask)
        s = oracle.two_sided_scores(sq_in, sq_out, qn_in, qn_out, kq["bits"], kq["norms"])[0]
        assert s == pytest.approx(sign * (qn_in * n16[0] + qn_out * n16[1]), rel=1e-14)


def test_two_sided_scores_identity_projection_page_vectors():
    """S = I tiled 4x (m = 32, d = 8) on the page's vectors: the sign agreement of q and k counted
    by hand, times |q| |k|16 / 8."""
    g = golden("page1_one_bit_keys.json")
    q = np.array(g["query_on"])
    S = tiled_identity(8, 32)
    for kv in g["keys"].values():
        kq = oracle.quantize_key_vectors(np.array([kv]), S, np.zeros((0, 8)), [])
        sq_in, sq_out = oracle.project_query(q, S, np.zeros((0, 8)), [])
        s = oracle.two_sided_scores(sq_in, sq_out, float(np.linalg.norm(q)), 0.0, kq["bits"], kq["norms"])[0]
        agree = sum(1 if (a >= 0) == (b >= 0) else -1 for a, b in zip(q, kv))
        assert s == pytest.approx(np.linalg.norm(q) * float(np.float16(np.linalg.norm(kv))) * agree / 8, rel=1e-13)
    # the 'on' query agrees with 'cat' on all but dimension 5 (0.05 vs 0.04: same sign) -> all 8
    assert sum((a >= 0) == (b >= 0) for a, b in zip(q, g["keys"]["cat"])) == 8


def test_decode_attention_estimator_switch():
    """The decode reference routes to the two scorers; an unknown estimator name is refused."""
    rng = np.random.default_rng(5)
    d, m, N = 16, 32, 9
    S = rng.standard_normal((m, d))
    K = rng.standard_normal((1, N, 1, d))
    kq = oracle.quantize_keys(K, S, np.zeros((0, d)), np.zeros((1, 0), np.int32))
    V = rng.standard_normal((1, 1, N, d))
    Q = rng.standard_normal((1, 2, d))
    one = oracle.decode_attention(Q, S, np.zeros((0, d)), np.zeros((1, 0), np.int32), kq["bits"], kq["norms"], N, V_f32=V)
    two = oracle.decode_attention(Q, S, np.zeros((0, d)), np.zeros((1, 0), np.int32), kq["bits"], kq["norms"], N, V_f32=V,
                                  estimator="two_sided")
    for hq in range(2):
        sq_in, sq_out = oracle.project_query(Q[0, hq], S, np.zeros((0, d)), [])
        bits, norms = kq["bits"][0, 0], kq["norms"][0, 0]
        assert np.array_equal(one["scores"][0, hq], oracle.estimator_scores(sq_in, sq_out, bits, norms))
        assert np.array_equal(two["scores"][0, hq],
                              oracle.two_sided_scores(sq_in, sq_out, np.linalg.norm(Q[0, hq]), 0.0, bits, norms))
    with pytest.raises(ValueError):
        oracle.decode_attention(Q, S, np.zeros((0, d)), np.zeros((1, 0), np.int32), kq["bits"], kq["norms"], N,
                                V_f32=V, estimator="cosine")


def test_rotate_sign_identity_is_norm_times_signs():
    """R = I: the page's reconstructed key, norm x signs scaled to the key's norm, dotted with q."""
    g = golden("page1_one_bit_keys.json")
    q = np.array(g["query_on"])
    K = np.array(list(g["keys"].values()))
    s = oracle.rotate_sign_scores(q, K, np.eye(8))
    for i, kv in enumerate(K):
        khat = np.linalg.norm(kv) * np.sign(kv) / math.sqrt(8)
        assert np.linalg.norm(khat) == pytest.approx(np.linalg.norm(kv), rel=1e-15)
        assert s[i] == pytest.approx(q @ khat, rel=1e-14)


def test_rotate_sign_closed_forms():
    """q = k scores ||k|| ||R k||_1 / sqrt(d); permuting or negating rows of R changes no score; and
    the one-sided estimator with S = sqrt(2d/pi) R gives the same scores up to the fp16 key norm."""
    rng = np.random.default_rng(8)
    d = 64
    R = si.random_rotation(3, d)
    assert np.allclose(R @ R.T, np.eye(d), atol=1e-12)
    K = rng.standard_normal((5, d))
    q = rng.standard_normal(d)
    s_kk = oracle.rotate_sign_scores(K[0], K[:1], R)[0]
    assert s_kk == pytest.approx(np.linalg.norm(K[0]) * np.abs(R @ K[0]).sum() / math.sqrt(d), rel=1e-13)
    # permuting and negating rows of R changes no score (the reconstruction's terms are reordered)
    P = np.eye(d)[rng.permutation(d)] * np.where(rng.random(d) < 0.5, -1.0, 1.0)[:, None]
    assert np.allclose(oracle.rotate_sign_scores(q, K, P @ R), oracle.rotate_sign_scores(q, K, R), rtol=1e-12)
    S = math.sqrt(2 * d / math.pi) * R
    kq = oracle.quantize_key_vectors(K, S, np.zeros((0, d)), [])
    sq_in, sq_out = oracle.project_query(q, S, np.zeros((0, d)), [])
    one = oracle.estimator_scores(sq_in, sq_out, kq["bits"], kq["norms"])
    ref = oracle.rotate_sign_scores(q, K, R)
    scale = np.linalg.norm(K, axis=1) * np.abs(R @ q).sum() / math.sqrt(d)
    assert np.all(np.abs(one - ref) <= 2 ** -11 * scale)


# ----------------------------------------------------------------------------- exact attention

def test_exact_attention_page_examples_and_closed_forms():
    """Unquantized attention (reporting reference): the page's dot product Q . K_cat = 16.203
    ("How Attention Computes a Score"); with two keys scoring 12.83 and 12.23 the weights are the
    page's [0.65, 0.35] and the output its 0.65 V_cat + 0.35 V_mat ("Why Truncation Kills", "Keys
    Select. Values Deliver."); one key returns its value; equal scores return the mean value; and an
    explicit loop over the softmax definition on random inputs."""
    g = golden("page1_one_bit_keys.json")
    q = np.array(g["query_on"])
    k_cat, v_cat, v_mat = (np.array(g["keys"]["cat"]), np.array(g["values"]["cat"]), np.array(g["values"]["mat"]))
    # keys {k_cat, 0} with one-hot values: the first output channel is the softmax weight of cat,
    # logistic(sm_scale * Q . K_cat); the page rounds each of its 8 products to 3 decimals (<= 0.004)
    sm = 0.1
    w_cat = oracle.exact_attention(q, np.stack([k_cat, np.zeros(8)]), np.eye(2), sm)[0]
    dot = math.log(w_cat / (1.0 - w_cat)) / sm
    assert dot == pytest.approx(g["score_on_cat_printed"], abs=4e-3)
    # one key: the softmax weight is 1
    np.testing.assert_allclose(oracle.exact_attention(q, k_cat[None], v_cat[None], 0.37), v_cat, rtol=0, atol=1e-15)
    # two keys along q with the page's scores 12.83 and 12.23 (sm_scale 1)
    K2 = np.stack([12.83 * q / (q @ q), 12.23 * q / (q @ q)])
    out = oracle.exact_attention(q, K2, np.stack([v_cat, v_mat]), 1.0)
    w = g["softmax_correct"]["weights_printed"]
    np.testing.assert_allclose(out, w[0] * v_cat + w[1] * v_mat, atol=0.006 * np.abs(v_cat - v_mat).max())
    wa = 1.0 / (1.0 + math.exp(-(12.83 - 12.23)))
    np.testing.assert_allclose(out, wa * v_cat + (1 - wa) * v_mat, rtol=0, atol=1e-13)
    # equal scores: every key orthogonal to q gives the mean of the values
    rng = np.random.default_rng(11)
    V = rng.standard_normal((9, 8))
    qo = np.zeros(8)
    qo[0] = 1.0
    Ko = rng.standard_normal((9, 8))
    Ko[:, 0] = 0.0
    np.testing.assert_allclose(oracle.exact_attention(qo, Ko, V, 3.0), V.mean(axis=0), rtol=0, atol=1e-14)
    # the definition written out as loops: scores <q, k_t>, scaled, max-subtracted exponentials
    K = rng.standard_normal((13, 8))
    V = rng.standard_normal((13, 8))
    qr = rng.standard_normal(8)
    sm = 0.6
    z = [sm * sum(qr[c] * K[t, c] for c in range(8)) for t in range(13)]
    mz = max(z)
    e = [math.exp(x - mz) for x in z]
    ref = [sum(e[t] * V[t, c] for t in range(13)) / sum(e) for c in range(8)]
    np.testing.assert_allclose(oracle.exact_attention(qr, K, V, sm), ref, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- batch and head routing

def test_batch_and_kv_head_routing():
    """Several sequences, KV heads and query heads per KV head (B = 3, Hkv = 2, g = 3), with a
    different outlier channel set per KV head.  Query head hq reads KV head hq // g: heads 0, 1, 2 read
    KV head 0 and heads 3, 4, 5 read KV head 1 (written out below, not computed).  Pinned three ways:
      * values: every value vector of (b, h) is the constant c[b, h], so the output of (b, hq) is
        exactly c[b, KV head of hq] whatever the scores are;
      * keys: the keys of (b, h) live on the outlier channels of KV head h only, so their inlier norm
        is 0, their inlier bits are all 1 (sign(0) = +1) and their outlier norm is the key's norm;
      * scores: each (b, hq) equals the single-head estimator on the projection of its own query
        with its KV head's outlier set, over that KV head's keys."""
    B, Hkv, g, N, d, m, m_out = 3, 2, 3, 11, 16, 32, 32
    Hq = Hkv * g
    kv_of = [0, 0, 0, 1, 1, 1]
    oidx = np.array([[1, 6], [9, 14]], dtype=np.int32)
    rng = np.random.default_rng(21)
    S_in, S_out = rng.standard_normal((m, d)), rng.standard_normal((m_out, d))
    K = np.zeros((B, N, Hkv, d))
    for h in range(Hkv):
        K[:, :, h, oidx[h]] = rng.standard_normal((B, N, 2)) * 3.0
    c = np.array([[1.0 + b + 0.25 * h for h in range(Hkv)] for b in range(B)])      # fp16-exact constants
    V = np.broadcast_to(c[:, None, :, None], (B, N, Hkv, d)).astype(np.float32)
    Q = rng.standard_normal((B, Hq, d))

    kq = oracle.quantize_keys(K, S_in, S_out, oidx)
    vq = oracle.quantize_values(V, 2)
    for b in range(B):
        for h in range(Hkv):
            assert np.all(kq["norms"][b, h, :, 0] == 0)
            full = np.linalg.norm(K[b, :, h, :], axis=1)
            np.testing.assert_array_equal(kq["norms"][b, h, :, 1], oracle.fp16(full))
            assert np.all(kq["bits"][b, h, :, : m // 32] == 0xFFFFFFFF)
            # the unit equals the single-vector quantizer on its own keys and outlier set
            r = oracle.quantize_key_vectors(K[b, :, h, :], S_in, S_out, oidx[h])
            np.testing.assert_array_equal(kq["bits"][b, h], r["bits"])

    res = oracle.decode_attention(Q, S_in, S_out, oidx, kq["bits"], kq["norms"], N, codes=vq["codes"],
                                  meta=vq["meta"], nbits=2)
    for b in range(B):
        for hq in range(Hq):
            h = kv_of[hq]
            np.testing.assert_allclose(res["out"][b, hq], c[b, h], rtol=0, atol=1e-13)
            sq_in, sq_out = oracle.project_query(Q[b, hq], S_in, S_out, oidx[h])
            np.testing.assert_array_equal(res["scores"][b, hq],
                                          oracle.estimator_scores(sq_in, sq_out, kq["bits"][b, h], kq["norms"][b, h]))
    # the head routing is what distinguishes the KV heads here: a swap of the two heads' data changes
    # every output, so the check above cannot pass by accident
    assert np.all(c[:, 0] != c[:, 1])
