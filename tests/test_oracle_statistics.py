"""Monte-Carlo pins of the oracle's estimator over random Gaussian JL matrices (no GPU).

The QJL summary ("Approach", "Surprising findings") states that quantizing one side of the JL
projection to signs gives an unbiased inner-product estimate, while quantizing both sides estimates
an angle-based quantity instead.  These tests check the oracle's estimator against those statements
and against its exact variance, which follows from E[X] = <q,k> and E[X^2] = (pi/2)|q|^2|k|^2 for
X = sqrt(pi/2) |k| <s,q> sign<s,k>, s ~ N(0, I):  Var(score) = ((pi/2)|q|^2|k|^2 - <q,k>^2) / m.
S is drawn in true fp64 here (bf16 rounding of S would add a bias of order 2^-9).
"""
import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si

D = 128


def _scores(q, k, m, m_out, ch, draws, seed):
    out = np.empty(draws)
    for r in range(draws):
        S_in = si.gaussian(seed, (m, D), r, 0)
        S_out = si.gaussian(seed, (m_out, D), r, 1)
        kq = oracle.quantize_key_vectors(k[None, :], S_in, S_out, ch)
        sq_in, sq_out = oracle.project_query(q, S_in, S_out, ch)
        out[r] = oracle.estimator_scores(sq_in, sq_out, kq["bits"], kq["norms"])[0]
    return out


def _var(q, k, m):
    return (math.pi / 2 * (q @ q) * (k @ k) - (q @ k) ** 2) / m


def _pair(seed, cos):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal(D)
    u = rng.standard_normal(D)
    u -= (u @ k) / (k @ k) * k
    q = cos * k / np.linalg.norm(k) + math.sqrt(1 - cos * cos) * u / np.linalg.norm(u)
    return q * 1.3, k * 0.8


@pytest.mark.parametrize("cos", [0.6, -0.3])
def test_one_sided_estimator_is_unbiased_with_the_exact_variance(cos):
    q, k = _pair(21, cos)
    m, draws = 256, 3000
    s = _scores(q, k, m, 0, [], draws, seed=500)
    true = q @ k
    var = _var(q, k, m)
    z = (s.mean() - true) / math.sqrt(var / draws)
    assert abs(z) < 5, z
    ratio = s.var(ddof=1) / var
    assert 0.9 < ratio < 1.1, ratio
    # a wrong constant would be far outside: 1/m instead of sqrt(pi/2)/m shifts the mean by 20%
    assert abs(true * (1 - math.sqrt(2 / math.pi))) / math.sqrt(var / draws) > 20


def test_outlier_split_estimator_is_unbiased_with_summed_variance():
    q, k = _pair(22, 0.5)
    ch = [5, 40, 90, 127]
    k[ch] *= 20.0
    q[ch] += 0.5                      # some query mass on the outlier channels
    m = m_out = 128
    draws = 3000
    s = _scores(q, k, m, m_out, ch, draws, seed=600)
    mask = np.zeros(D, bool)
    mask[ch] = True
    qi, ki, qo, ko = q * ~mask, k * ~mask, q * mask, k * mask
    var = _var(qi, ki, m) + _var(qo, ko, m_out)
    z = (s.mean() - q @ k) / math.sqrt(var / draws)
    assert abs(z) < 5, z
    ratio = s.var(ddof=1) / var
    assert 0.9 < ratio < 1.1, ratio
    # the masked query matters: an unmasked query would have this (different) variance
    var_unmasked = _var(q, ki, m) + _var(q, ko, m_out)
    assert abs(var_unmasked / var - 1) > 0.25


def test_error_shrinks_like_one_over_sqrt_m():
    q, k = _pair(23, 0.4)
    rms = []
    for m in (64, 1024):
        s = _scores(q, k, m, 0, [], 600, seed=700 + m)
        rms.append(math.sqrt(np.mean((s - q @ k) ** 2)))
    assert rms[1] / rms[0] == pytest.approx(0.25, rel=0.2)


def test_two_sided_sign_estimator_is_biased_toward_the_angle():
    """Signs on both sides: E[sign<s,q> sign<s,k>] = 1 - 2 theta / pi, not cos(theta)."""
    q, k = _pair(24, 0.7)
    theta = math.acos((q @ k) / (np.linalg.norm(q) * np.linalg.norm(k)))
    est = np.mean([oracle.two_sided_estimate(q, k, si.gaussian(800, (256, D), r)) for r in range(400)])
    assert est == pytest.approx(1 - 2 * theta / math.pi, abs=0.01)
    assert abs(est - math.cos(theta)) > 0.1


def test_two_sided_decode_scores_average_to_the_angle_term():
    """The decode-path two-sided scorer (with the outlier split) averages, over Gaussian JL draws, to
    sum over parts of ||q_part|| ||k_part||16 (1 - 2 theta_part / pi)."""
    q, k = _pair(31, 0.6)
    ch = [5, 77, 100]
    mask = oracle.outlier_mask(D, ch)
    qi, qo, ki, ko = q * (1 - mask), q * mask, k * (1 - mask), k * mask

    def angle(a, b):
        return math.acos(float(a @ b) / (np.linalg.norm(a) * np.linalg.norm(b)))

    vals = []
    for r in range(300):
        S_in, S_out = si.gaussian(900, (256, D), r, 0), si.gaussian(900, (256, D), r, 1)
        kq = oracle.quantize_key_vectors(k[None, :], S_in, S_out, ch)
        sq_in, sq_out = oracle.project_query(q, S_in, S_out, ch)
        vals.append(oracle.two_sided_scores(sq_in, sq_out, np.linalg.norm(qi), np.linalg.norm(qo), kq["bits"],
                                            kq["norms"])[0])
    n16 = kq["norms"][0].astype(np.float64)
    expect = (np.linalg.norm(qi) * n16[0] * (1 - 2 * angle(qi, ki) / math.pi)
              + np.linalg.norm(qo) * n16[1] * (1 - 2 * angle(qo, ko) / math.pi))
    scale = np.linalg.norm(qi) * n16[0] + np.linalg.norm(qo) * n16[1]
    assert np.mean(vals) == pytest.approx(expect, abs=0.01 * scale)
    # and not the inner product: the bias of the two-sided estimate is visible
    assert abs(np.mean(vals) - q @ k) > 0.05 * scale
