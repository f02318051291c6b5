"""The value quantizer's shortcuts around IEEE division, checked on the CPU in float32 (no GPU).

The kernels take step = fp16((max - min) / L) from the product with fl32(1 / L), and the quotients
(v - min16) / step from the product with a reciprocal of step that is within one ulp, each with a
fallback to the correctly rounded division when the shortcut's result lies close to a rounding
boundary.  These tests model both shortcuts in numpy float32 (the reciprocal perturbed by -1, 0 and
+1 ulp, the worst cases of v_rcp_f32) and check that, wherever no fallback is taken, they give the
same fp16 step and the same code as the correctly rounded divisions of the recipe.
"""
import numpy as np
import pytest

F32 = np.float32


def _step_shortcut(rng_: np.ndarray, L: int):
    z = rng_ * F32(F32(1.0) / F32(L))
    dropped = z.view(np.uint32) & np.uint32(0x1FFF)
    fallback = (z < F32(2.0 ** -14)) | ((dropped >= 0x1000 - 4) & (dropped <= 0x1000 + 4))
    return z, fallback


@pytest.mark.parametrize("L", [3, 7, 15])
def test_step_product_rounds_like_the_division(L):
    g = np.random.default_rng(L)
    # ranges over many binades, plus ranges built to sit on fp16 halfway points after the division
    r = (g.uniform(0.5, 1.0, 400_000) * 2.0 ** g.integers(-16, 14, 400_000)).astype(F32)
    halves = (np.float16(g.uniform(1e-3, 100.0, 50_000)).astype(F32).view(np.uint32) + np.uint32(0x1000)).view(F32)
    tie_r = np.concatenate([halves * F32(L), np.nextafter(halves * F32(L), F32(np.inf)), np.nextafter(halves * F32(L), F32(0))]).astype(F32)
    for rng_ in (r, tie_r):
        exact16 = (rng_ / F32(L)).astype(np.float16)
        z, fallback = _step_shortcut(rng_, L)
        assert np.array_equal(z[~fallback].astype(np.float16).view(np.uint16), exact16[~fallback].view(np.uint16))
    normal = r / F32(L) >= F32(2.0 ** -13)                       # steps in the fp16 normal range
    assert np.mean(_step_shortcut(r[normal], L)[1]) < 0.002      # the fallback stays rare there


@pytest.mark.parametrize("L", [3, 7, 15])
@pytest.mark.parametrize("ulps", [-1, 0, 1])
def test_code_product_rounds_like_the_division(L, ulps):
    g = np.random.default_rng(100 + L)
    n = 300_000
    step = np.float16(g.uniform(1e-3, 4.0, n)).astype(F32)
    # values uniform over the levels, and values a few ulps around the halfway points k + 1/2
    x_uni = (g.uniform(-0.3, L + 0.3, n) * step).astype(F32)
    k = g.integers(-1, L + 1, n).astype(F32)
    mid = ((k + F32(0.5)) * step).astype(F32)
    x_tie = (mid.view(np.int32) + g.integers(-3, 4, n).astype(np.int32)).view(F32)
    rcp = (F32(1.0) / step).astype(F32)
    rcp = (rcp.view(np.int32) + np.int32(ulps)).view(F32)
    for x in (x_uni, x_tie):
        exact = np.clip(np.rint(x / step), 0, L)
        y = (x * rcp).astype(F32)
        r = np.rint(y)
        fallback = np.abs(y - r) >= F32(0.5) - F32(2.0 ** -20) * F32(L + 2)
        fast = np.clip(r, 0, L)
        assert np.array_equal(fast[~fallback], exact[~fallback])
    assert np.mean(np.abs((x_uni * rcp) - np.rint(x_uni * rcp)) >= 0.5 - 2.0 ** -20 * (L + 2)) < 1e-3


def _fma32(a, b, c):
    """float32 fused multiply-add: the float32 product is exact in float64, so the sum is rounded once to
    float64 and once more to float32 (a second rounding that can move the result by one float32 ulp in
    rare halfway cases, well inside the margin the kernels keep)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F32)


@pytest.mark.parametrize("L", [3, 7, 15])
@pytest.mark.parametrize("ulps", [-1, 0, 1])
def test_offset_product_rounds_like_the_division(L, ulps):
    """The kernels' fast path: y = fma(v, rcp, fma(-base, rcp, 1/2)), code = floor(y) clamped to [0, L],
    unless the fraction of y lies within 2^-20 (L + 2 + |base rcp|) of 0 or 1 (then the divide)."""
    g = np.random.default_rng(200 + L + ulps)
    n = 300_000
    step = np.float16(g.uniform(1e-3, 4.0, n)).astype(F32)
    # minima over many magnitudes, both signs (an offset far from zero stresses the offset's rounding)
    base = np.float16(g.choice([-1.0, 1.0], n) * g.uniform(0.0, 1.0, n) * 10.0 ** g.integers(-3, 4, n)).astype(F32)
    v_uni = (base + (g.uniform(-0.3, L + 0.3, n) * step)).astype(F32)
    k = g.integers(-1, L + 1, n).astype(F32)
    mid = (base + (k + F32(0.5)) * step).astype(F32)
    v_tie = (mid.view(np.int32) + g.integers(-3, 4, n).astype(np.int32)).view(F32)
    rcp = (F32(1.0) / step).astype(F32)
    rcp = (rcp.view(np.int32) + np.int32(ulps)).view(F32)
    off = _fma32(-base, rcp, np.full(n, 0.5, F32))
    marg = (F32(2.0 ** -20) * (F32(L + 2) + np.abs((base * rcp).astype(F32)))).astype(F32)
    for v in (v_uni, v_tie):
        v = np.where(np.isfinite(v), v, base)           # an integer nudge of a zero midpoint is not a value
        exact = np.clip(np.rint(((v - base).astype(F32) / step).astype(F32)), 0, L)
        y = _fma32(v, rcp, off)
        f = (y - np.floor(y)).astype(F32)
        fallback = (f <= marg) | (f >= F32(1.0) - marg)
        fast = np.floor(np.clip(y, F32(0.0), F32(L + 0.5)))
        assert np.array_equal(fast[~fallback], exact[~fallback])
        # every exact tie takes the divide
        ties = ((v - base).astype(F32) / step).astype(F32) - np.floor(((v - base).astype(F32) / step).astype(F32)) == F32(0.5)
        assert np.all(fallback[ties & (exact > 0) & (exact < L)])
    moderate = np.abs(base / step) < 64
    y = _fma32(v_uni, rcp, off)
    f = y - np.floor(y)
    assert np.mean(((f <= marg) | (f >= 1 - marg))[moderate]) < 1e-3   # the divide stays rare
