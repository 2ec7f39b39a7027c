"""Pins of the DDIM oracle: closed forms, schedule structure, a published value.

* the schedule: beta_0 = 0.00085 exactly gives alpha_bar_0; the betas read back
  from consecutive alpha_bar ratios have square roots in arithmetic
  progression from sqrt(0.00085) to sqrt(0.012) (the scaled_linear shape);
  SD's terminal value sqrt(alpha_bar_999) = 0.068265 as published by Lin et
  al., "Common Diffusion Noise Schedules and Sample Steps are Flawed" (WACV
  2024), section 3.1;
* the step: x_t built from a known (x0, eps) by the forward marginal returns
  x0 and returns x_prev on the forward marginal at t - 333 with the same eps;
* the pyramid: every window at its own t recovers its own x0.

A sign error, a swapped sqrt(a) / sqrt(1-a), a wrong step length or a wrong
window index each fail one of these.
"""

import numpy as np
import pytest

from oracle import (
    sd_scaled_linear_alphas_cumprod,
    ddim_coefficients,
    ddim_step,
    pyramid_ddim_step,
)

AB = sd_scaled_linear_alphas_cumprod()


def test_table_and_step_length_match_the_pages(pages_constants):
    ts = pages_constants["timesteps"]
    step = pages_constants["step_length"]
    assert len(ts) == pages_constants["num_inference_steps"]
    assert all(a - b == step for a, b in zip(ts, ts[1:]))
    assert ts[-1] == 0 and ts[0] == len(AB) - 1


def test_alpha_bar_zero_is_one_minus_beta_start():
    assert abs(AB[0] - (1.0 - 0.00085)) <= 1e-15


def test_betas_follow_scaled_linear_shape():
    betas = np.empty_like(AB)
    betas[0] = 1.0 - AB[0]
    betas[1:] = 1.0 - AB[1:] / AB[:-1]
    r = np.sqrt(betas)
    assert abs(r[0] - np.sqrt(0.00085)) <= 1e-12
    assert abs(r[-1] - np.sqrt(0.012)) <= 1e-10
    step = (np.sqrt(0.012) - np.sqrt(0.00085)) / 999.0
    assert np.max(np.abs(np.diff(r) - step)) <= 1e-9
    assert np.all(np.diff(AB) < 0)


def test_published_terminal_value():
    # Lin et al. (WACV 2024), section 3.1: SD's schedule ends at sqrt(alpha_bar_T) = 0.068265
    assert abs(np.sqrt(AB[999]) - 0.068265) <= 1e-6


@pytest.mark.parametrize("t", [999, 666, 333])
def test_recovers_x0_and_lands_on_forward_marginal(t):
    rng = np.random.default_rng(t)
    x0 = rng.standard_normal((4, 8, 8))
    eps = rng.standard_normal((4, 8, 8))
    x_t = np.sqrt(AB[t]) * x0 + np.sqrt(1 - AB[t]) * eps
    x_prev, x0_hat = ddim_step(x_t, eps, t, 333, AB)
    assert np.max(np.abs(x0_hat - x0)) <= 1e-10
    target = np.sqrt(AB[t - 333]) * x0 + np.sqrt(1 - AB[t - 333]) * eps
    assert np.max(np.abs(x_prev - target)) <= 1e-10


def test_t0_window_keeps_its_sample_and_emits_x0():
    rng = np.random.default_rng(0)
    x0 = rng.standard_normal(64)
    eps = rng.standard_normal(64)
    x_t = np.sqrt(AB[0]) * x0 + np.sqrt(1 - AB[0]) * eps
    x_prev, x0_hat = ddim_step(x_t, eps, 0, 333, AB)
    assert np.max(np.abs(x_prev - x_t)) <= 1e-14  # alpha_prev = alpha_bar_0 = alpha_t
    assert np.max(np.abs(x0_hat - x0)) <= 1e-12
    # with final alpha 1 the t=0 step lands on x0 itself
    x_prev1, _ = ddim_step(x_t, eps, 0, 333, AB, final_alpha_cumprod=1.0)
    assert np.max(np.abs(x_prev1 - x0)) <= 1e-12


def test_coefficient_form_matches_direct_form():
    rng = np.random.default_rng(1)
    x_t = rng.standard_normal(100)
    eps = rng.standard_normal(100)
    for t in (999, 666, 333, 0, 500, 1):
        a, b, c, d = ddim_coefficients(t, 333, AB)
        xp, x0 = ddim_step(x_t, eps, t, 333, AB)
        assert np.max(np.abs(a * x_t + b * eps - xp)) <= 1e-12
        assert np.max(np.abs(c * x_t + d * eps - x0)) <= 1e-12


def test_pyramid_windows_each_use_their_own_timestep():
    rng = np.random.default_rng(2)
    ts = [999, 666, 333, 0]
    x0 = rng.standard_normal((16, 4, 8, 8))
    eps = rng.standard_normal((16, 4, 8, 8))
    x_t = np.empty_like(x0)
    for w, t in enumerate(ts):
        blk = slice(4 * w, 4 * w + 4)
        x_t[blk] = np.sqrt(AB[t]) * x0[blk] + np.sqrt(1 - AB[t]) * eps[blk]
    x_prev, x0_out = pyramid_ddim_step(x_t, eps, ts, 333, AB, emit_window=3)
    assert np.max(np.abs(x0_out - x0[12:16])) <= 1e-12
    for w, t in enumerate(ts[:3]):
        blk = slice(4 * w, 4 * w + 4)
        target = np.sqrt(AB[t - 333]) * x0[blk] + np.sqrt(1 - AB[t - 333]) * eps[blk]
        assert np.max(np.abs(x_prev[blk] - target)) <= 1e-10
    assert np.max(np.abs(x_prev[12:16] - x_t[12:16])) <= 1e-14
    # rolled order: the emitted window can sit in any slot
    x_prev_r, x0_r = pyramid_ddim_step(x_t[::-1].copy(), eps[::-1].copy(), ts[::-1], 333, AB, emit_window=0)
    assert x0_r is not None and x0_r.shape == (4, 4, 8, 8)


def test_known_coefficient_values():
    # x0 at t=999 is a strongly cancelling combination: C = 1/sqrt(a) ~ 14.65
    a, b, c, d = ddim_coefficients(999, 333, AB)
    assert abs(c - 1 / 0.068265) < 5e-3
    assert abs(c * c - 1 - d * d) <= 1e-9  # (1/sqrt a)^2 - ((1-a)/a) = 1
    a0, b0, c0, d0 = ddim_coefficients(0, 333, AB)
    assert a0 == pytest.approx(1.0, abs=1e-15) and abs(b0) <= 1e-15


def test_out_of_range_timestep_rejected():
    with pytest.raises(ValueError):
        ddim_step(np.zeros(2), np.zeros(2), 1000, 333, AB)
