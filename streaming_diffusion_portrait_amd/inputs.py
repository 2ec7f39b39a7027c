"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method: it only draws random numbers
(NumPy's PCG64 through ``SeedSequence.spawn``) and lays them out in the shapes
of the streaming pyramid's workloads.  Both the HIP path and the CPU oracle
consume what it returns; neither is imported here.

Shapes follow the SD1.5 UNet used by PersonaLive at 512x512 (latent 64x64):
transformer levels of 64^2 / 32^2 / 16^2 / 8^2 tokens with 320 / 640 / 1280 /
1280 channels and 8 heads; a 16-frame batch of 4 windows x 4 frames; a
512-dimensional motion embedding.
"""

import numpy as np

# The 16 transformer layers of the SD1.5 denoiser in execution order
# (down 64^2 x2, 32^2 x2, 16^2 x2; mid 8^2; up 16^2 x3, 32^2 x3, 64^2 x3),
# named as in the fused engine's explicit reference inputs.
SD15_LAYERS = (
    ("d00", 4096, 320), ("d01", 4096, 320),
    ("d10", 1024, 640), ("d11", 1024, 640),
    ("d20", 256, 1280), ("d21", 256, 1280),
    ("m", 64, 1280),
    ("u10", 256, 1280), ("u11", 256, 1280), ("u12", 256, 1280),
    ("u20", 1024, 640), ("u21", 1024, 640), ("u22", 1024, 640),
    ("u30", 4096, 320), ("u31", 4096, 320), ("u32", 4096, 320),
)


def rng_stream(seed, n_streams, index):
    """Generator number ``index`` of ``n_streams`` spawned from ``seed``."""
    return np.random.default_rng(np.random.SeedSequence(int(seed)).spawn(int(n_streams))[int(index)])


def normal(seed, n_streams, index, shape, dtype=np.float32):
    """N(0, 1) samples of ``shape`` from one spawned stream, cast to ``dtype``."""
    x = rng_stream(seed, n_streams, index).standard_normal(size=shape, dtype=np.float32)
    return x.astype(dtype, copy=False)


def attention_layer(seed, F, L, C, m, q_gain=1.0):
    """Seeded fp16 inputs of one reference-bank attention layer.

    Returns a dict with ``q, k_self, v_self`` ``[F, L, C]`` and ``bank_k,
    bank_v`` lists of ``1 + m`` arrays ``[L, C]`` (the reference entry and m
    anchors), all float16 drawn as N(0, 1) float32 and rounded to nearest.
    ``q_gain`` scales Q before rounding (a "peaky logits" stress input).
    """
    n = 3 + 2 * (1 + m)
    q = normal(seed, n, 0, (F, L, C))
    if q_gain != 1.0:
        q = q * np.float32(q_gain)
    out = {
        "q": q.astype(np.float16),
        "k_self": normal(seed, n, 1, (F, L, C), np.float16),
        "v_self": normal(seed, n, 2, (F, L, C), np.float16),
        "bank_k": [normal(seed, n, 3 + 2 * j, (L, C), np.float16) for j in range(1 + m)],
        "bank_v": [normal(seed, n, 4 + 2 * j, (L, C), np.float16) for j in range(1 + m)],
    }
    return out


def ddim_pile(seed, shape=(16, 4, 64, 64)):
    """Seeded fp32 (x_t, eps) for the pile: both N(0, 1), window-major."""
    return normal(seed, 2, 0, shape), normal(seed, 2, 1, shape)


def motion_bank(seed, n, D=512, nq=1, sigma_range=(0.5, 1.0)):
    """Seeded motion bank and queries.

    The bank holds ``n`` N(0, 1) entries of dimension D.  Each query is a bank
    entry (chosen uniformly) plus sigma * z with z ~ N(0, 1) and sigma ~
    U[sigma_range], so its distances straddle the drift threshold.
    Returns float32 ``(bank [n, D], queries [nq, D], source_index [nq])``.
    """
    g = rng_stream(seed, 1, 0)
    bank = g.standard_normal((n, D), dtype=np.float32)
    src = g.integers(0, n, size=nq)
    sig = g.uniform(sigma_range[0], sigma_range[1], size=nq).astype(np.float32)
    z = g.standard_normal((nq, D), dtype=np.float32)
    queries = bank[src] + sig[:, None] * z
    return bank, queries.astype(np.float32), src


def round_m(seed):
    """The round's anchor count m in 0..3, one seeded draw."""
    return int(rng_stream(seed, 2, 1).integers(0, 4))
