"""Pins of the motion-bank and pile oracles.

Motion: brute force with pure-Python sums, a library distance routine, exact
ties at the threshold, Pythagorean distances, identical vectors and duplicate
bank entries (lowest index wins).

Pile: a simulation of many rounds checks the structural claims of the
streaming pyramid: every window is evaluated at 999, 666, 333, 0 in four
consecutive rounds and then leaves, windows leave first-in first-out, four
frames leave per round and the forward always sees 16 frames.
"""

import math

import numpy as np
import pytest

from oracle import motion_bank_min_l2, PyramidPile


def test_motion_brute_force():
    rng = np.random.default_rng(0)
    bank = rng.standard_normal((4, 512))
    qs = rng.standard_normal((6, 512))
    dist, arg, flag = motion_bank_min_l2(qs, bank, 17.0)
    for i in range(6):
        ds = [math.sqrt(sum((qs[i, k] - bank[j, k]) ** 2 for k in range(512))) for j in range(4)]
        j = min(range(4), key=lambda jj: (ds[jj], jj))
        assert arg[i] == j
        assert abs(dist[i] - ds[j]) <= 1e-12 * ds[j]
        assert flag[i] == (ds[j] > 17.0)


def test_motion_matches_library_cdist():
    scipy_spatial = pytest.importorskip("scipy.spatial")
    rng = np.random.default_rng(1)
    bank = rng.standard_normal((3, 512))
    qs = rng.standard_normal((5, 512)) * 0.7
    dist, arg, _ = motion_bank_min_l2(qs, bank)
    ref = scipy_spatial.distance.cdist(qs, bank)
    assert np.array_equal(arg, ref.argmin(axis=1))
    assert np.max(np.abs(dist - ref.min(axis=1))) <= 1e-12


def test_motion_exact_tie_is_not_an_exceed(pages_constants):
    thr = pages_constants["motion_threshold"]
    bank = np.zeros((2, 512))
    bank[1] = 100.0
    q = np.zeros((1, 512))
    q[0, 7] = 17.0
    dist, arg, flag = motion_bank_min_l2(q, bank, thr)
    assert dist[0] == 17.0 and arg[0] == 0 and not flag[0]
    q[0, 7] = 17.0 + 2.0 ** -10
    assert motion_bank_min_l2(q, bank, thr)[2][0]


def test_motion_pythagorean_distance():
    bank = np.zeros((1, 512))
    q = np.zeros((1, 512))
    q[0, 100], q[0, 300] = 8.0, 15.0
    dist, _, flag = motion_bank_min_l2(q, bank, 17.0)
    assert dist[0] == 17.0 and not flag[0]
    q[0, 300] = 15.001
    assert motion_bank_min_l2(q, bank, 17.0)[2][0]


def test_motion_identical_and_duplicates():
    rng = np.random.default_rng(2)
    e = rng.standard_normal(512)
    bank = np.stack([e + 30.0, e, e, e - 30.0])
    dist, arg, flag = motion_bank_min_l2(e[None], bank)
    assert dist[0] == 0.0 and arg[0] == 1 and not flag[0]
    far = np.stack([e + 1.0, e + 1.0])
    assert motion_bank_min_l2(e[None], far)[1][0] == 0


def test_motion_single_query_vector_and_errors():
    d, a, f = motion_bank_min_l2(np.ones(512), np.zeros((1, 512)))
    assert d.shape == (1,) and abs(d[0] - math.sqrt(512)) <= 1e-12 and f[0]
    with pytest.raises(ValueError):
        motion_bank_min_l2(np.ones((1, 4)), np.ones((1, 5)))


def test_pile_windows_walk_the_table_and_leave_fifo(pages_constants):
    ts = pages_constants["timesteps"]
    fpw = pages_constants["frames_per_window"]
    pile = PyramidPile(ts, fpw)
    assert pile.frames() == pages_constants["prefill_frames"]
    seen = {}
    emitted = []
    for r in range(12):
        evaluated, out = pile.round()
        assert len(evaluated) * fpw == pages_constants["batch_frames"]
        assert [t for _, t in evaluated] == ts[::-1]  # oldest (t=0) first, newest at 999
        for wid, t in evaluated:
            seen.setdefault(wid, []).append(t)
        assert out is not None  # the prefilled pile emits from the first round
        emitted.append(out)
        assert pile.frames() == pages_constants["prefill_frames"]
    assert emitted == sorted(emitted)  # first in, first out
    for wid in range(3, 3 + 9):  # windows that entered at 999 and left
        assert seen[wid] == list(ts)


def test_pile_without_prefill_first_emits_after_four_rounds():
    pile = PyramidPile((999, 666, 333, 0), 4, prefill=False)
    outs = [pile.round()[1] for _ in range(6)]
    assert outs[:3] == [None, None, None]
    assert outs[3:] == [0, 1, 2]
