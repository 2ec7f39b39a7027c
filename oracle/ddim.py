"""Oracle: the per-window DDIM step of the streaming pyramid, in fp64.

Test infrastructure only (see the package docstring).

PersonaLive write-up, section "它解决什么" (specification): DDIM with 4 steps,
epsilon prediction, fp16 model, 512x512.  Section "流式金字塔去噪": the
timestep table is fixed to 999, 666, 333, 0 and the scheduler's step length is
set to 333, so every window moves from its own t to ``t - 333``; the window
leaving the queue hands ``pred_original_sample`` (the x0 prediction) to the
VAE rather than the last sample.

Readings where the pages are silent (listed in the design notes):

* noise schedule: Stable Diffusion 1.5's ``scaled_linear`` betas,
  ``beta = linspace(sqrt(0.00085), sqrt(0.012), 1000) ** 2``,
  ``alpha_bar = cumprod(1 - beta)`` (the base models are SD checkpoints);
* eta = 0 (deterministic DDIM), no clipping of x0;
* when ``t - step_len < 0`` the "previous" alpha_bar is ``final_alpha_cumprod``,
  by default ``alpha_bar[0]`` (SD's scheduler keeps alpha_bar[0] rather than
  1 there).  That window's x_prev is discarded anyway; its x0 is the output.

The step itself (plain DDIM with eta = 0)::

    x0     = (x_t - sqrt(1 - a_t) * eps) / sqrt(a_t)
    x_prev = sqrt(a_prev) * x0 + sqrt(1 - a_prev) * eps
"""

import numpy as np


def sd_scaled_linear_alphas_cumprod(num_train_timesteps=1000, beta_start=0.00085, beta_end=0.012):
    """alpha_bar_t for SD's scaled_linear schedule, t = 0..T-1, in fp64."""
    betas = np.linspace(np.sqrt(beta_start), np.sqrt(beta_end), num_train_timesteps, dtype=np.float64) ** 2
    return np.cumprod(1.0 - betas)


def _alpha_pair(t, step_len, alphas_cumprod, final_alpha_cumprod):
    a = np.asarray(alphas_cumprod, dtype=np.float64)
    if not 0 <= t < a.shape[0]:
        raise ValueError("timestep out of range")
    a_t = a[t]
    prev = t - step_len
    if prev >= 0:
        a_prev = a[prev]
    else:
        a_prev = a[0] if final_alpha_cumprod is None else float(final_alpha_cumprod)
    return a_t, a_prev


def ddim_coefficients(t, step_len=333, alphas_cumprod=None, final_alpha_cumprod=None):
    """(A, B, C, D) with x_prev = A*x_t + B*eps and x0 = C*x_t + D*eps.

    Obtained by expanding the two DDIM formulas in the module docstring.
    """
    if alphas_cumprod is None:
        alphas_cumprod = sd_scaled_linear_alphas_cumprod()
    a_t, a_prev = _alpha_pair(t, step_len, alphas_cumprod, final_alpha_cumprod)
    c = 1.0 / np.sqrt(a_t)
    d = -np.sqrt(1.0 - a_t) / np.sqrt(a_t)
    a = np.sqrt(a_prev) * c
    b = np.sqrt(a_prev) * d + np.sqrt(1.0 - a_prev)
    return a, b, c, d


def ddim_step(x_t, eps, t, step_len=333, alphas_cumprod=None, final_alpha_cumprod=None):
    """One deterministic DDIM step for one window: returns (x_prev, x0) in fp64."""
    if alphas_cumprod is None:
        alphas_cumprod = sd_scaled_linear_alphas_cumprod()
    a_t, a_prev = _alpha_pair(t, step_len, alphas_cumprod, final_alpha_cumprod)
    x_t = np.asarray(x_t, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    x0 = (x_t - np.sqrt(1.0 - a_t) * eps) / np.sqrt(a_t)
    x_prev = np.sqrt(a_prev) * x0 + np.sqrt(1.0 - a_prev) * eps
    return x_prev, x0


def pyramid_ddim_step(x_t, eps, t_windows, step_len=333, alphas_cumprod=None,
                      final_alpha_cumprod=None, emit_window=None):
    """The pyramid's DDIM update over a pile of W windows.

    ``x_t`` and ``eps`` have a leading axis that splits evenly into
    ``W = len(t_windows)`` windows (e.g. 16 frames = 4 windows x 4 frames);
    window w holds the contiguous block ``w`` and steps from ``t_windows[w]``.
    Returns ``(x_prev, x0)``: ``x_prev`` has x_t's shape; ``x0`` is the
    emitted window's x0 prediction (shape of one window) or ``None`` when
    ``emit_window`` is None.
    """
    x_t = np.asarray(x_t, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    W = len(t_windows)
    if x_t.shape != eps.shape or x_t.shape[0] % W:
        raise ValueError("x_t / eps shapes must match and split into W windows")
    per = x_t.shape[0] // W
    x_prev = np.empty_like(x_t)
    x0_out = None
    for w in range(W):
        blk = slice(w * per, (w + 1) * per)
        xp, x0 = ddim_step(x_t[blk], eps[blk], int(t_windows[w]), step_len,
                           alphas_cumprod, final_alpha_cumprod)
        x_prev[blk] = xp
        if emit_window is not None and w == emit_window:
            x0_out = x0
    return x_prev, x0_out
