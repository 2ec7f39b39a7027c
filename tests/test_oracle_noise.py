"""Pins of the pile-roll oracle (window noise, staircase prefill, motion interpolation).

Philox-4x64-10 is pinned to NumPy's own Philox bit generator (a library
implementation of the same published generator); the normal transform by
the inverse relations of Box-Muller and a Kolmogorov-Smirnov test; the
prefill by the DDIM closed form (recovering the reference from the noised
window); the interpolation by its end points and constant spacing.
"""

import numpy as np
import pytest
from scipy import stats

from oracle import (philox4x64, uniform24, window_noise, noise_at, staircase_prefill, lerp_points,
                    ddim_step, sd_scaled_linear_alphas_cumprod)

MASK = (1 << 64) - 1


def plus_one(counter):
    """256-bit counter + 1 (little-endian words), as NumPy's generator steps it."""
    c = list(counter)
    for i in range(4):
        c[i] = (c[i] + 1) & MASK
        if c[i] != 0:
            break
    return c


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((5, 7, 0, 3), (11, 13)),
    ((MASK, 1, 2, 3), (2**63 + 5, 99)),          # carry into word 1
    ((MASK, MASK, MASK, 0), (MASK, MASK)),       # carry into word 3
    ((123456789, 0, 0, 0), (2024, 7)),
])
def test_philox_matches_numpy_generator(counter, key):
    # NumPy advances the counter before producing each block of four words
    bg = np.random.Philox(counter=np.array(counter, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    raw = [int(x) for x in bg.random_raw(8)]
    c1 = plus_one(counter)
    c2 = plus_one(c1)
    assert raw[:4] == philox4x64(c1, key)
    assert raw[4:] == philox4x64(c2, key)


def test_philox_rounds_matter():
    # a dropped round or a wrong key schedule would change the output
    assert philox4x64((1, 2, 3, 4), (5, 6), rounds=10) != philox4x64((1, 2, 3, 4), (5, 6), rounds=9)
    assert philox4x64((1, 2, 3, 4), (5, 6)) != philox4x64((1, 2, 3, 4), (6, 5))


def test_uniform24_range_and_exactness():
    assert uniform24(0) == 2.0 ** -24
    assert uniform24(MASK) == 1.0
    assert uniform24((1 << 40) - 1) == 2.0 ** -24          # low 40 bits ignored
    assert uniform24(1 << 40) == 2.0 * 2.0 ** -24
    u = uniform24(0x9E3779B97F4A7C15)
    assert np.float32(u) == u                                  # exact in fp32


def test_window_noise_inverts_to_generator_words():
    seed, wid, n = 31, 4, 64
    z = window_noise(seed, wid, n)
    for blk in range(n // 4):
        w = philox4x64((blk, 0, 0, 0), (seed, wid))
        u = [uniform24(x) for x in w]
        for p in range(2):
            z0, z1 = z[4 * blk + 2 * p], z[4 * blk + 2 * p + 1]
            # radius from the first word of the pair, angle from the second
            assert np.isclose(z0 * z0 + z1 * z1, -2.0 * np.log(u[2 * p]), rtol=1e-12, atol=1e-12)
            ang = np.arctan2(z1, z0) % (2 * np.pi)
            assert np.isclose(ang, (2 * np.pi * u[2 * p + 1]) % (2 * np.pi), rtol=0, atol=1e-9) or \
                np.isclose(abs(ang - 2 * np.pi * u[2 * p + 1]), 2 * np.pi, atol=1e-9)


def test_window_noise_is_standard_normal():
    z = window_noise(2024, 0, 1 << 15)
    n = z.size
    assert abs(z.mean()) < 5.0 / np.sqrt(n)
    assert abs(z.var() - 1.0) < 5.0 * np.sqrt(2.0 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    # windows and seeds give independent-looking streams
    z2 = window_noise(2024, 1, 1 << 12)
    z3 = window_noise(2025, 0, 1 << 12)
    assert abs(np.corrcoef(z[: 1 << 12], z2)[0, 1]) < 0.08
    assert abs(np.corrcoef(z[: 1 << 12], z3)[0, 1]) < 0.08


def test_window_noise_ragged_length_is_a_prefix():
    full = window_noise(9, 2, 40)
    assert np.array_equal(window_noise(9, 2, 37), full[:37])
    assert np.array_equal(noise_at(9, 2, [39, 0, 17, 17]), full[[39, 0, 17, 17]])


def test_staircase_prefill_recovers_reference_through_ddim():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(256)
    seed, W, step = 17, 3, 333
    pile = staircase_prefill(ref, seed, W, step)
    a = sd_scaled_linear_alphas_cumprod()
    for w in range(W):
        t = w * step
        eps = window_noise(seed, w, ref.size)
        # the noised window is exactly the forward marginal: DDIM's x0 with the
        # true noise gives the reference back (closed form)
        _, x0 = ddim_step(pile[w], eps, t, step)
        assert np.allclose(x0, ref, rtol=0, atol=1e-9)
        assert np.allclose(pile[w], np.sqrt(a[t]) * ref + np.sqrt(1 - a[t]) * eps, atol=0)
    # t = 0 keeps the reference almost clean: alpha_bar_0 = 1 - beta_0 = 0.99915
    assert np.allclose(pile[0], ref, atol=0.2)


def test_lerp_points_end_points_and_spacing():
    a = np.array([0.0, 1.0, -2.0, 5.0])
    b = np.array([12.0, 1.0, 10.0, -7.0])
    pts = lerp_points(a, b, 12)
    assert pts.shape == (12, 4)
    assert np.array_equal(pts[0], a)
    d = np.diff(pts, axis=0)
    assert np.allclose(d, (b - a) / 12.0, atol=1e-12)
    assert np.allclose(pts[-1] + (b - a) / 12.0, b, atol=1e-12)  # the dropped 13th point is b
