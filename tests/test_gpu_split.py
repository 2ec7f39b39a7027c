"""GPU parity of the key-axis split (the small levels' launches at d = 160).

A launch that holds fewer waves than the GPU has SIMDs splits its key tiles
among several workgroups per (head, frame, query tile); each writes its
partial output, offset and row sum to the caller's workspace and a combine
kernel merges them (the softmax of the whole key axis).  The bank's 1x..4x
length (PersonaLive write-up, section TensorRT 融合) makes the key axis 5x the
query count at the 16^2 and 8^2 levels.  Each case is compared element by
element with the fp64 oracle, with the split and with the single-pass
kernels; split boundaries fall between and inside segments and on ragged
tiles, and one case forces the exact re-run inside a split.
"""

import zlib

import numpy as np
import pytest

from oracle import refbank_attention
from streaming_diffusion_portrait_amd import inputs
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


def rand16(rng, *shape, gain=1.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(gain)).astype(np.float16)


def make(name, F, L, H, segspec, q_gain=1.0):
    """segspec: list of (len, shared, k_gain); d = 160."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    C = H * 160
    q = rand16(rng, F, L, C, gain=q_gain)
    segs = []
    for ln, shared, kg in segspec:
        shape = (ln, C) if shared else (F, ln, C)
        segs.append((rand16(rng, *shape, gain=kg), rand16(rng, *shape), shared))
    return q, segs


def run(B, q, segs, H, workspace=None):
    out = B.refbank_attn(dev(q), [(dev(k), dev(v)) for k, v, _ in segs], H, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # (name, F, L, H, segspec): the launch must leave CUs idle, so these are
    # few-frame launches with long key axes; the boundaries fall inside
    # segments and next to ragged tiles
    ("ragged segments, one tile per split", 1, 64, 2,
     [(100, False, 1.0), (64, True, 1.0), (30, True, 1.0), (129, True, 1.0), (600, True, 1.0), (150, True, 1.0)]),
    ("one frame, 41 splits", 1, 40, 1, [(64, False, 1.0), (1024, True, 1.0), (1024, True, 1.0), (512, True, 1.0)]),
    ("query tail beyond one block, two tiles per split", 2, 57, 2, [(57, False, 1.0), (512, True, 1.0), (512, True, 1.0)]),
    ("16 frames x 8 heads, boundary inside a segment", 16, 64, 8,
     [(64, False, 1.0), (256, True, 1.0), (512, True, 1.0), (256, True, 1.0)]),
    ("16 frames x 8 heads, ragged tiles", 16, 64, 8,
     [(70, False, 1.0), (100, True, 1.0), (600, True, 1.0), (330, True, 1.0)]),
]


@pytest.mark.parametrize("name,F,L,H,segspec", CASES, ids=[c[0] for c in CASES])
def test_split_matches_oracle_and_single_pass(B, name, F, L, H, segspec):
    say("split", name)
    q, segs = make(name, F, L, H, segspec)
    assert B.workspace_size(F, L, H, 160, [s[0] for s in segspec]) > 0, "the case must split"
    ref = refbank_attention(q, segs, H)
    got = run(B, q, segs, H)
    assert_attn_close(got, ref, name + " (split)")
    single = run(B, q, segs, H, workspace=False)
    assert_attn_close(single, ref, name + " (single pass)")


def test_exact_rerun_inside_a_split(B):
    # 16 frames x 8 heads at 64 rows, 18 key tiles: two splits of nine.  In the
    # first, tile 0 has tiny scores (the frozen offset is low) and tile 1 large
    # ones: that split's frozen offset overflows and it re-runs with exact maxima
    say("split exact re-run")
    F, L, H = 16, 64, 8
    spec = [(64, False, 0.01), (64, True, 6.0), (1024, True, 1.0)]
    q, segs = make("split rerun", F, L, H, spec)
    n = B.workspace_size(F, L, H, 160, [s[0] for s in spec])
    assert n == F * H * 2 * L * 162 * 4  # two splits
    ref = refbank_attention(q, segs, H)
    got = run(B, q, segs, H)
    e = assert_attn_close(got, ref, "split re-run")
    assert e["norm_rel"] <= 2e-3, e


def test_level_8x8_full(B):
    # the 8^2 level of the round at m = 3 (5 key tiles: no split; the 64-row
    # two-wave configuration), in full against the oracle
    say("8^2 level full")
    lay = inputs.attention_layer(3, 16, 64, 1280, 3)
    segs = [(lay["k_self"], lay["v_self"], False)] + [(k, v, True) for k, v in zip(lay["bank_k"], lay["bank_v"])]
    assert B.workspace_size(16, 64, 8, 160, [64] * 5) == 0
    assert_attn_close(run(B, lay["q"], segs, 8), refbank_attention(lay["q"], segs, 8), "8^2")


def test_one_frame_levels_split(B):
    # the round's 16^2 and 8^2 shapes for a single frame (the 4x bank): the
    # launches that split, sampled against the oracle
    for L in (256, 64):
        say("one-frame split, L =", L)
        lay = inputs.attention_layer(60 + L, 1, L, 1280, 3)
        segs = [(lay["k_self"], lay["v_self"], False)] + [(k, v, True) for k, v in zip(lay["bank_k"], lay["bank_v"])]
        assert B.workspace_size(1, L, 8, 160, [L] * 5) > 0
        got = run(B, lay["q"], segs, 8)
        assert_attn_close(got, refbank_attention(lay["q"], segs, 8), f"one frame L={L}")


def test_caller_workspace_reused(B):
    # one caller-owned workspace serves consecutive launches of different sizes
    say("split caller workspace")
    s1spec = [(64, False, 1.0), (600, True, 1.0), (600, True, 1.0)]
    s2spec = [(33, False, 1.0), (1100, True, 1.0)]
    q1, s1 = make("ws a", 2, 64, 2, s1spec)
    q2, s2 = make("ws b", 1, 33, 2, s2spec)
    n1 = B.workspace_size(2, 64, 2, 160, [x[0] for x in s1spec])
    n2 = B.workspace_size(1, 33, 2, 160, [x[0] for x in s2spec])
    assert n1 > 0 and n2 > 0
    ws = torch.full((max(n1, n2),), 255, dtype=torch.uint8, device="cuda")  # stale contents must not matter
    assert_attn_close(run(B, q1, s1, 2, workspace=ws), refbank_attention(q1, s1, 2), "ws a")
    assert_attn_close(run(B, q2, s2, 2, workspace=ws), refbank_attention(q2, s2, 2), "ws b")
