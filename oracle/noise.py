"""Oracle: the pile's device-side roll -- fresh window noise, the staircase
prefill and the motion interpolation of the first frames -- in fp64.

Test infrastructure only (see the package docstring).

PersonaLive write-up, section "流式金字塔去噪": each round a new window enters
the pile at t = 999 and the window that reached t = 0 leaves; the TensorRT
section lists the fused graph's ``new_noise`` input (the new window's
latents) and ``bind()``, which points each round's outputs at the next
round's inputs so the rolling state never leaves device memory.  Section
"首帧怎么办": the queue starts pre-filled with 12 frames of staircase noise
(three windows at three noise levels) and the pose and expression inputs of
those frames are linear interpolations, 12 + 1 points from the reference's to
the first driving frame's, the last point dropped.

The pages do not say how the noise is drawn.  Reading: a counter-based
generator, so that any window's noise can be produced on the device from
(seed, window id) alone.  The generator is Philox-4x64 with 10 rounds
(Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
3", SC 2011), written out here from that definition; normals come from the
Box-Muller transform.  The exact recipe both sides follow:

* key = (seed, window id); element i of a window uses counter
  (i // 4, 0, 0, 0) and output word i % 4;
* each 64-bit word x gives u = ((x >> 40) + 1) / 2**24, in (0, 1];
* words (0, 1) give z0 = r cos(2 pi u1), z1 = r sin(2 pi u1) with
  r = sqrt(-2 ln u0); words (2, 3) give z2, z3 the same way.

Staircase prefill (reading, parity of the content unpinned by the pages):
slot w holds the window at t = w * step_len, the reference latent noised to
that level, ``sqrt(a_t) * ref + sqrt(1 - a_t) * noise(seed, w)``.

Motion interpolation: point k of n + 1 evenly spaced points from a to b is
``a + (b - a) * k / n``; the first n points are kept.
"""

import numpy as np

from .ddim import sd_scaled_linear_alphas_cumprod

_MASK = (1 << 64) - 1
# Philox-4x64 round multipliers and Weyl key increments (the published constants)
_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B


def philox4x64(counter, key, rounds=10):
    """Philox-4x64-R of one 256-bit counter under a 128-bit key (Python ints).

    Each round multiplies words 0 and 2 by the two constants, keeps both
    halves of the 128-bit products and mixes them with the other two words
    and the key; the key is bumped by the Weyl constants before every round
    but the first.
    """
    c = [int(v) & _MASK for v in counter]
    k = [int(v) & _MASK for v in key]
    for r in range(rounds):
        if r:
            k = [(k[0] + _W0) & _MASK, (k[1] + _W1) & _MASK]
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> 64, p0 & _MASK
        hi1, lo1 = p1 >> 64, p1 & _MASK
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return c


def uniform24(word):
    """The (0, 1] uniform of a 64-bit word: its top 24 bits, plus one, over 2**24."""
    return ((int(word) >> 40) + 1) / float(1 << 24)


def window_noise(seed, window_id, n):
    """N(0, 1) noise of one window: n values, fp64, by the recipe above."""
    out = np.empty(n, dtype=np.float64)
    for blk in range((n + 3) // 4):
        z = window_noise_block(seed, window_id, blk)
        for j in range(4):
            i = 4 * blk + j
            if i < n:
                out[i] = z[j]
    return out


def noise_at(seed, window_id, indices):
    """Elements ``indices`` of window_noise(seed, window_id, ...), fp64 (for sampled checks)."""
    idx = np.asarray(indices, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.float64)
    cache = {}
    for j, i in enumerate(idx.tolist()):
        blk = i // 4
        if blk not in cache:
            cache[blk] = window_noise_block(seed, window_id, blk)
        out[j] = cache[blk][i % 4]
    return out


def window_noise_block(seed, window_id, blk):
    """The four normals of elements 4*blk .. 4*blk+3 (the recipe in the module docstring)."""
    w = philox4x64((blk, 0, 0, 0), (seed, window_id))
    u = [uniform24(x) for x in w]
    z = []
    for a, b in ((u[0], u[1]), (u[2], u[3])):
        r = np.sqrt(-2.0 * np.log(a))
        z += [r * np.cos(2.0 * np.pi * b), r * np.sin(2.0 * np.pi * b)]
    return z


def staircase_prefill(ref, seed, n_windows, step_len=333, alphas_cumprod=None):
    """[n_windows, n] fp64: slot w = ref noised to t = w * step_len with noise(seed, w)."""
    if alphas_cumprod is None:
        alphas_cumprod = sd_scaled_linear_alphas_cumprod()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    out = np.empty((n_windows, ref.size), dtype=np.float64)
    for w in range(n_windows):
        a = float(alphas_cumprod[w * step_len])
        out[w] = np.sqrt(a) * ref + np.sqrt(1.0 - a) * window_noise(seed, w, ref.size)
    return out


def lerp_points(a, b, n):
    """[n, ...] fp64: points k = 0 .. n-1 of n + 1 evenly spaced points from a to b."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.stack([a + (b - a) * (k / n) for k in range(n)])
