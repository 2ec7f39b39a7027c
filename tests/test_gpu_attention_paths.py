"""GPU parity of pl_refbank_attn on inputs chosen to drive each path of the kernel.

The kernel evaluates the first key tile with exact block maxima, then freezes
the softmax offset; key sequences made only of whole 64-key tiles run a
software-pipelined loop, others a tile-by-tile loop; a frozen offset that a
later score exceeds by 16 or more (log2 units) makes the workgroup start over
with exact maxima on every tile; offsets beyond +-1024 never freeze.  Every
case here is compared element by element with the fp64 oracle.
"""

import zlib

import numpy as np
import pytest

from oracle import refbank_attention
from _helpers import assert_attn_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_diffusion_portrait_amd import binding
    binding.load()
    return binding


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(B, q, segs, H):
    out = B.refbank_attn(dev(q), [(dev(k), dev(v)) for k, v, _ in segs], H)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def rand16(rng, *shape, gain=1.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(gain)).astype(np.float16)


def make(name, d, F, L, H, segspec, q_gain=1.0):
    """segspec: list of (len, shared, k_gain)."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    C = H * d
    q = rand16(rng, F, L, C, gain=q_gain)
    segs = []
    for ln, shared, kg in segspec:
        shape = (ln, C) if shared else (F, ln, C)
        segs.append((rand16(rng, *shape, gain=kg), rand16(rng, *shape), shared))
    return q, segs


# Whole-tile key sequences: 1..5 tiles (pipeline prologue, drain and the
# four-slot ring wrapping), several segments (the copy side crossing segment
# boundaries, including one-tile segments), more than one frame.
FULL = [
    ("d40 one tile", 40, 2, 130, 2, [(64, False, 1.0)]),
    ("d40 two tiles", 40, 2, 130, 2, [(64, False, 1.0), (64, True, 1.0)]),
    ("d40 three tiles", 40, 1, 257, 2, [(192, False, 1.0)]),
    ("d40 five tiles three segs", 40, 3, 300, 1, [(128, False, 1.0), (64, True, 1.0), (128, True, 1.0)]),
    ("d40 ring wraps", 40, 1, 256, 2, [(256, False, 1.0), (320, True, 1.0), (64, True, 1.0)]),
    ("d32 four tiles", 32, 2, 200, 2, [(128, False, 1.0), (128, True, 1.0)]),
    ("d32 six segs", 32, 1, 128, 2, [(64, False, 1.0), (64, True, 1.0), (64, True, 1.0), (64, True, 1.0),
                                       (64, True, 1.0), (128, True, 1.0)]),
    ("d80 full", 80, 2, 100, 1, [(128, False, 1.0), (192, True, 1.0)]),
    ("d160 full", 160, 1, 70, 2, [(64, False, 1.0), (128, True, 1.0)]),
]


@pytest.mark.parametrize("name,d,F,L,H,segspec", FULL, ids=[c[0] for c in FULL])
def test_whole_tiles(B, name, d, F, L, H, segspec):
    say("attn path", name)
    q, segs = make(name, d, F, L, H, segspec)
    got = run_gpu(B, q, segs, H)
    assert_attn_close(got, refbank_attention(q, segs, H), name)


# Scores that rise far above the first tile's maximum: the frozen offset
# overflows fp16 and the workgroup must recompute with exact maxima.
RISING = [
    ("d40 rising full", 40, 2, 128, 2, [(128, False, 0.01), (128, True, 10.0)]),
    ("d40 rising ragged", 40, 2, 100, 2, [(70, False, 0.01), (90, True, 10.0)]),
    ("d32 rising", 32, 1, 128, 2, [(64, False, 0.01), (192, True, 12.0)]),
    ("d80 rising", 80, 1, 64, 2, [(64, False, 0.01), (128, True, 8.0)]),
    ("d160 rising", 160, 1, 64, 1, [(64, False, 0.01), (64, True, 6.0)]),
]


@pytest.mark.parametrize("name,d,F,L,H,segspec", RISING, ids=[c[0] for c in RISING])
def test_rising_scores_restart(B, name, d, F, L, H, segspec):
    say("attn path", name)
    q, segs = make(name, d, F, L, H, segspec)
    # the inputs must really exceed the first tile's maximum by >= 16 log2 units
    d_ = d
    scale = d_ ** -0.5 * np.log2(np.e)
    first = np.asarray(segs[0][0], np.float64)
    later = np.asarray(segs[1][0], np.float64)
    q0 = np.asarray(q[0][:, :d_], np.float64)
    f0 = first[0][:, :d_] if first.ndim == 3 else first[:, :d_]
    l0 = later[0][:, :d_] if later.ndim == 3 else later[:, :d_]
    gap = (q0 @ l0.T).max(axis=1) * scale - (q0 @ f0[:64].T).max(axis=1) * scale
    assert gap.max() > 16.0, gap.max()
    got = run_gpu(B, q, segs, H)
    assert_attn_close(got, refbank_attention(q, segs, H), name)


# Offsets beyond +-1024 (log2 units): the offset never freezes, every tile is
# exact.  One key per row dominates by hundreds of log2 units, so the result is
# that key's value row and stays well conditioned.
HUGE = [
    ("d40 huge positive", 40, 1, 96, 2, 192, 40.0, 20.0, 40.0),
    ("d40 huge negative", 40, 1, 64, 1, 128, 40.0, -40.0, -30.0),
    ("d80 huge positive", 80, 1, 64, 1, 128, 30.0, 15.0, 30.0),
]


@pytest.mark.parametrize("name,d,F,L,H,lk,qg,kg,kstar", HUGE, ids=[c[0] for c in HUGE])
def test_huge_scores_exact_tiles(B, name, d, F, L, H, lk, qg, kg, kstar):
    say("attn path", name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    C = H * d
    u = np.ones(C, dtype=np.float32)
    q = np.broadcast_to(qg * u, (F, L, C)).astype(np.float16)
    k = np.broadcast_to(kg * u, (F, lk, C)).copy()
    jstar = int(rng.integers(64, lk))  # beyond the first tile: the exact path must move the offset
    k[:, jstar, :] = kstar
    k = k.astype(np.float16)
    v = rand16(rng, F, lk, C)
    segs = [(k, v, False)]
    scale = d ** -0.5 * np.log2(np.e)
    s = np.asarray(q[0][:, :d], np.float64) @ np.asarray(k[0][:, :d], np.float64).T * scale
    assert np.abs(s[:, :64].max(axis=1)).min() > 1024.0  # the first tile's offset cannot freeze
    got = run_gpu(B, q, segs, H)
    ref = refbank_attention(q, segs, H)
    assert np.allclose(ref[0], np.asarray(v[0][jstar], np.float64)[None, :], atol=1e-6)
    assert_attn_close(got, ref, name)


# One workgroup (256 query rows at d = 40) whose waves disagree about
# freezing: one wave's 64 rows have offsets far beyond +-1024 (they stay
# exact), the other waves' rows are ordinary.  The key sequence (8 whole
# tiles) is longer than the copy ring, so tiles are copied inside the loop;
# the workgroup must take one path for all of its waves.
MIXED = [("huge rows in the first wave", 0), ("huge rows in the last wave", 192)]


@pytest.mark.parametrize("name,row0", MIXED, ids=[c[0] for c in MIXED])
def test_mixed_offsets_in_one_workgroup(B, name, row0):
    say("attn path mixed offsets", name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    F, L, H, d, lk = 1, 256, 1, 40, 512
    q = rng.standard_normal((F, L, d), dtype=np.float32)
    q[:, row0:row0 + 64, :] = 40.0
    k = 20.0 + rng.standard_normal((F, lk, d), dtype=np.float32)
    jstar = int(rng.integers(64, lk))
    k[:, jstar, :] = 40.0
    q, k = q.astype(np.float16), k.astype(np.float16)
    v = rng.standard_normal((F, lk, d), dtype=np.float32).astype(np.float16)
    segs = [(k, v, False)]
    scale = d ** -0.5 * np.log2(np.e)
    s = np.asarray(q[0], np.float64) @ np.asarray(k[0], np.float64).T * scale
    m0 = s[:, :64].max(axis=1)
    assert np.abs(m0[row0:row0 + 64]).min() > 1024.0
    others = np.r_[0:row0, row0 + 64:L]
    assert np.abs(m0[others]).max() < 1024.0
    got = run_gpu(B, q, segs, H)
    assert_attn_close(got, refbank_attention(q, segs, H), name)
