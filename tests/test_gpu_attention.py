"""GPU parity of pl_refbank_attn against the fp64 oracle.

Small cases are compared element by element over the whole output; they span
several query and key tiles with ragged tails and every supported head
dimension.  The workload shapes (tiny, top 64^2, mid 32^2, low 16^2 / 8^2)
run at full size in the launch configuration the bench uses and are compared
on seeded samples of (frame, head, row) that the oracle computes one by one.
"""

import zlib

import numpy as np
import pytest

from oracle import refbank_attention
from streaming_diffusion_portrait_amd import inputs
from _helpers import assert_attn_close, attn_errors, say

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


def run_gpu(B, q, segs, H, scale=None):
    """segs: list of (k, v, shared) numpy fp16 arrays -> GPU output as numpy fp16."""
    dq = dev(q)
    dsegs = [(dev(k), dev(v)) for k, v, _ in segs]
    out = B.refbank_attn(dq, dsegs, H, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def rand16(rng, *shape, gain=1.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(gain)).astype(np.float16)


SMALL = [
    # (name, d, F, L, H, [(len, shared)], gain)
    ("d40 ragged NT1", 40, 3, 300, 2, [(300, False), (100, True), (37, True)], 1.0),
    ("d40 ragged NT4", 40, 2, 1100, 1, [(1100, False), (130, True)], 1.0),
    ("d40 peaky", 40, 2, 200, 2, [(200, False), (200, True)], 4.0),
    ("d80 ragged NT1", 80, 2, 130, 2, [(130, False), (64, True), (65, True), (1, True)], 1.0),
    ("d80 ragged NT2", 80, 2, 1030, 1, [(1030, False), (70, True)], 1.0),
    ("d160 ragged NT1", 160, 2, 70, 2, [(70, False), (33, True)], 1.0),
    ("d160 ragged NT2", 160, 1, 1025, 1, [(1025, False), (31, True), (32, True)], 1.0),
    # frames of at most 64 rows: two waves per query block, each with half of O^T's d tiles
    ("d160 small frame ragged", 160, 3, 37, 2, [(37, False), (100, True), (1, True)], 1.0),
    ("d160 small frame whole tiles", 160, 2, 64, 2, [(64, False), (128, True), (64, True)], 1.0),
    ("d32 ragged", 32, 2, 257, 2, [(257, False), (256, True), (5, True)], 1.0),
    ("d32 NT4", 32, 1, 1024, 2, [(1024, False), (1024, True)], 1.0),
    ("single key", 40, 2, 64, 2, [(1, False)], 1.0),
    ("one query row", 40, 2, 1, 2, [(1, False), (130, True)], 1.0),
    ("one query row, whole tiles", 80, 2, 1, 1, [(64, False), (128, True)], 1.0),
    ("bank only", 80, 3, 50, 1, [(77, True)], 1.0),
    # the most segments a call takes (8), per-frame and shared mixed: ragged ones
    # (tile-by-tile path) and whole tiles only (the pipelined path seeks across them)
    ("d40 eight ragged segments", 40, 2, 150, 2,
     [(150, False), (64, True), (1, True), (65, False), (128, True), (3, True), (64, False), (100, True)], 1.0),
    ("d40 eight whole segments", 40, 2, 128, 2,
     [(128, False), (64, True), (192, True), (64, False), (128, True), (64, True), (64, False), (256, True)], 1.0),
    ("d80 eight whole segments", 80, 2, 256, 1,
     [(256, False), (64, True), (128, True), (64, False), (64, True), (192, True), (64, False), (64, True)], 1.0),
    ("d160 eight ragged segments", 160, 2, 70, 1,
     [(70, False), (30, True), (64, True), (64, False), (1, True), (129, True), (7, False), (64, True)], 1.0),
]


@pytest.mark.parametrize("name,d,F,L,H,segspec,gain", SMALL, ids=[s[0] for s in SMALL])
def test_small_full_compare(B, name, d, F, L, H, segspec, gain):
    say("attn", name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    C = H * d
    q = rand16(rng, F, L, C, gain=gain)
    segs = []
    for ln, shared in segspec:
        shape = (ln, C) if shared else (F, ln, C)
        segs.append((rand16(rng, *shape), rand16(rng, *shape), shared))
    got = run_gpu(B, q, segs, H)
    ref = refbank_attention(q, segs, H)
    e = assert_attn_close(got, ref, name)
    assert e["norm_rel"] <= 2e-3, e


def test_strided_views_of_fused_qkv(B):
    say("attn strided qkv views")
    rng = np.random.default_rng(5)
    F, L, H, d = 2, 200, 2, 40
    C = H * d
    qkv = dev(rand16(rng, F, L, 3 * C))
    bank = dev(rand16(rng, 90, 2 * C))
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    bk, bv = bank[:, :C], bank[:, C:]
    out = torch.zeros(F, L + 3, C + 8, dtype=torch.float16, device="cuda")[:, :L, :C]
    B.refbank_attn(q, [(k, v), (bk, bv)], H, out=out)
    torch.cuda.synchronize()
    h = lambda t: t.cpu().numpy()
    ref = refbank_attention(h(q), [(h(k), h(v), False), (h(bk), h(bv), True)], H)
    assert_attn_close(h(out), ref, "strided")


@pytest.mark.parametrize("d", [40, 80, 160])
def test_short_context_strided_views(B, d):
    """The short-context kernel's row copies on strided views: Q a column slice of
    a fused [F, L, 3C] projection output, the expression tokens' K/V slices of one
    [F, 32, 2C] buffer, O written into a wider padded buffer."""
    say("attn short strided", d)
    rng = np.random.default_rng(50 + d)
    F, L, H = 2, 77, 2
    C = H * d
    qkv = dev(rand16(rng, F, L, 3 * C))
    kv = dev(rand16(rng, F, 32, 2 * C))
    q = qkv[..., :C]
    k, v = kv[..., :C], kv[..., C:]
    out = torch.zeros(F, L + 5, C + 16, dtype=torch.float16, device="cuda")
    view = out[:, :L, 8:8 + C]
    B.refbank_attn(q, [(k, v)], H, out=view)
    torch.cuda.synchronize()
    h = lambda t: t.cpu().numpy()
    ref = refbank_attention(h(q), [(h(k), h(v), False)], H)
    assert_attn_close(h(view), ref, f"short strided d{d}")
    # nothing outside the view was written
    rest = h(out).copy()
    rest[:, :L, 8:8 + C] = 0
    assert not rest.any()


def test_segment_order_does_not_matter(B):
    say("attn segment order")
    rng = np.random.default_rng(6)
    F, L, H, d = 2, 150, 2, 40
    C = H * d
    q = rand16(rng, F, L, C)
    segs = [(rand16(rng, F, L, C), rand16(rng, F, L, C), False),
            (rand16(rng, 90, C), rand16(rng, 90, C), True),
            (rand16(rng, 60, C), rand16(rng, 60, C), True)]
    a = run_gpu(B, q, segs, H)
    b = run_gpu(B, q, [segs[2], segs[0], segs[1]], H)
    ref = refbank_attention(q, segs, H)
    assert_attn_close(a, ref, "order a")
    assert_attn_close(b, ref, "order b")


def test_deterministic(B):
    say("attn determinism")
    lay = inputs.attention_layer(11, 4, 1024, 320, 1)
    segs = [(lay["k_self"], lay["v_self"], False)] + [(k, v, True) for k, v in zip(lay["bank_k"], lay["bank_v"])]
    a = run_gpu(B, lay["q"], segs, 8)
    b = run_gpu(B, lay["q"], segs, 8)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def _sampled_check(B, name, seed, F, L, C, H, m, n_pairs=6, n_rows=96):
    say("attn", name, f"F={F} L={L} C={C} H={H} m={m}")
    lay = inputs.attention_layer(seed, F, L, C, m)
    segs = [(lay["k_self"], lay["v_self"], False)] + [(k, v, True) for k, v in zip(lay["bank_k"], lay["bank_v"])]
    got = run_gpu(B, lay["q"], segs, H)
    assert np.all(np.isfinite(got))
    d = C // H
    rng = np.random.default_rng(seed + 1000)
    pairs = {(int(rng.integers(F)), int(rng.integers(H))) for _ in range(n_pairs)}
    pairs |= {(0, 0), (F - 1, H - 1)}
    worst = None
    for f, h in sorted(pairs):
        rows = np.unique(np.concatenate([rng.choice(L, size=min(n_rows, L), replace=False), [0, L - 1]]))
        ref = refbank_attention(lay["q"], segs, H, frames=[f], head_list=[h], rows=rows)[(f, h)]
        e = assert_attn_close(got[f][rows][:, h * d:(h + 1) * d], ref, f"{name} f={f} h={h}")
        worst = e if worst is None or e["max_abs"] > worst["max_abs"] else worst
    say("attn", name, "worst", worst)
    return got


def test_config_tiny_full(B):
    say("attn tiny full")
    lay = inputs.attention_layer(0, 16, 256, 64, 0)
    segs = [(lay["k_self"], lay["v_self"], False), (lay["bank_k"][0], lay["bank_v"][0], True)]
    got = run_gpu(B, lay["q"], segs, 2)
    ref = refbank_attention(lay["q"], segs, 2)
    assert_attn_close(got, ref, "tiny")


def test_config_top(B):
    _sampled_check(B, "top 64^2 d40", 1, 16, 4096, 320, 8, 0)


def test_config_top_stress_peaky(B):
    say("attn top peaky")
    lay = inputs.attention_layer(21, 16, 4096, 320, 0, q_gain=4.0)
    segs = [(lay["k_self"], lay["v_self"], False), (lay["bank_k"][0], lay["bank_v"][0], True)]
    got = run_gpu(B, lay["q"], segs, 8)
    rows = np.arange(0, 4096, 97)
    for f, h in [(0, 0), (7, 3), (15, 7)]:
        ref = refbank_attention(lay["q"], segs, 8, frames=[f], head_list=[h], rows=rows)[(f, h)]
        assert_attn_close(got[f][rows][:, h * 40:(h + 1) * 40], ref, f"peaky f={f} h={h}")


def test_config_mid(B):
    _sampled_check(B, "mid 32^2 d80 m3", 2, 16, 1024, 640, 8, 3)


def test_config_low_256(B):
    _sampled_check(B, "low 16^2 d160 m3", 3, 16, 256, 1280, 8, 3)


def test_config_low_64_full(B):
    say("attn low 8^2 full")
    lay = inputs.attention_layer(3, 16, 64, 1280, 3)
    segs = [(lay["k_self"], lay["v_self"], False)] + [(k, v, True) for k, v in zip(lay["bank_k"], lay["bank_v"])]
    got = run_gpu(B, lay["q"], segs, 8)
    ref = refbank_attention(lay["q"], segs, 8)
    assert_attn_close(got, ref, "low 8^2")


def test_max_bank_top_level(B):
    # the largest key axis of the round: 64^2 with three anchors (Lk = 20480)
    _sampled_check(B, "top 64^2 d40 m3", 31, 16, 4096, 320, 8, 3, n_pairs=3, n_rows=48)


def test_zero_queries_mean_of_values_at_scale(B):
    # property that holds at any size: Q = 0 gives the mean of all values
    say("attn zero q property")
    lay = inputs.attention_layer(41, 2, 4096, 320, 1)
    q = np.zeros_like(lay["q"])
    segs = [(lay["k_self"], lay["v_self"], False)] + [(k, v, True) for k, v in zip(lay["bank_k"], lay["bank_v"])]
    got = run_gpu(B, q, segs, 8)
    for f in range(2):
        vals = np.concatenate([lay["v_self"][f].astype(np.float64)] + [v.astype(np.float64) for v in lay["bank_v"]])
        mean = vals.mean(axis=0)
        err = np.abs(got[f].astype(np.float64) - mean[None, :])
        assert err.max() <= 1e-2 and err.mean() <= 1e-3, (err.max(), err.mean())


# ---- bounded-context key lists (sink + sliding window, PR-Sink) -------------------
def _chunk_stream(seed, n_chunks, L, C):
    rng = np.random.default_rng(seed)
    f16 = lambda *s: rng.standard_normal(s, dtype=np.float32).astype(np.float16)
    return [(f16(L, C), f16(L, C)) for _ in range(n_chunks)], (f16(L, C), f16(L, C))


@pytest.mark.parametrize("scheme,d,L,H", [("sink_window", 40, 192, 2), ("sink_window", 80, 100, 1),
                                          ("pr_sink", 40, 128, 2), ("pr_sink", 160, 64, 1)])
def test_bounded_context_segments(B, scheme, d, L, H):
    """A chunk's attention over the key list a bounded-context scheme picks:
    current chunk + cached chunks + reference, one call, against the oracle."""
    from streaming_diffusion_portrait_amd.context import sink_window_ids, pr_sink_ids, context_segments
    say("bounded context", scheme, d, L, H)
    C = H * d
    chunks, ref = _chunk_stream(zlib.crc32(scheme.encode()) + d, 12, L, C)
    current = 11
    rng = np.random.default_rng(d)
    q = rng.standard_normal((1, L, C), dtype=np.float32).astype(np.float16)
    if scheme == "sink_window":
        ids = sink_window_ids(current)
    else:
        # dynamic sink: the earlier chunk whose pose embedding is nearest (GPU min-L2 check)
        # among four candidate chunks (3..6), the way the motion bank is searched
        poses = rng.standard_normal((current, 512), dtype=np.float32)
        query_pose = poses[5] + 0.01 * rng.standard_normal(512, dtype=np.float32)
        _, am, _ = B.motion_bank_min_l2(dev(query_pose), dev(poses[3:7]), 17.0)
        ids = pr_sink_ids(current, dynamic=3 + int(am.cpu().numpy()[0]))
        assert 5 in ids
    cur = (chunks[current][0][None], chunks[current][1][None])
    segs_np = context_segments(cur, {i: chunks[i] for i in range(current)}, ids, ref)
    assert len(segs_np) <= 8
    segs = [(k, v, k.ndim == 2) for k, v in segs_np]
    got = run_gpu(B, q, segs, H)
    assert_attn_close(got, refbank_attention(q, segs, H), f"{scheme} d={d}")


# ---- short contexts: the expression (32 tokens per frame) and CLIP (1 token) ----
SHORT = [
    # (name, d, F, L, H, seglen, shared)
    ("expr d40 small", 40, 3, 300, 2, 32, False),
    ("expr d80 small", 80, 2, 130, 2, 32, False),
    ("expr d160 small", 160, 2, 70, 1, 32, False),
    ("expr d32 small", 32, 2, 257, 2, 32, False),
    ("clip d40 small", 40, 2, 100, 2, 1, True),
    ("ctx 64 d40", 40, 2, 1000, 1, 64, True),
    ("ctx 50 d80 ragged rows", 80, 1, 37, 2, 50, False),
    ("one query row d40", 40, 3, 1, 2, 32, False),
    ("one query row d160 clip", 160, 1, 1, 1, 1, True),
    ("expr d40 8 heads, 33 rows", 40, 2, 33, 8, 32, False),
]


@pytest.mark.parametrize("name,d,F,L,H,seglen,shared", SHORT, ids=[c[0] for c in SHORT])
def test_short_context_full(B, name, d, F, L, H, seglen, shared):
    say("attn short", name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    C = H * d
    q = rand16(rng, F, L, C)
    shape = (seglen, C) if shared else (F, seglen, C)
    segs = [(rand16(rng, *shape), rand16(rng, *shape), shared)]
    got = run_gpu(B, q, segs, H)
    ref = refbank_attention(q, segs, H)
    assert_attn_close(got, ref, name)
    if seglen == 1:  # one key: every output row is that key's value row
        v = segs[0][1].astype(np.float64)
        assert np.allclose(got.astype(np.float64), np.broadcast_to(v, got.shape), atol=1e-3)


@pytest.mark.parametrize("L,C", [(4096, 320), (1024, 640), (256, 1280), (64, 1280)])
def test_short_context_workload_sampled(B, L, C):
    """Expression cross-attention at each level: 16 frames, 8 heads, 32 keys per frame."""
    say("attn expression level", L, C)
    H, F = 8, 16
    rng = np.random.default_rng(L + C)
    q = rand16(rng, F, L, C)
    segs = [(rand16(rng, F, 32, C), rand16(rng, F, 32, C), False)]
    got = run_gpu(B, q, segs, H)
    d = C // H
    rows = np.unique(np.concatenate([rng.choice(L, size=min(64, L), replace=False), [0, L - 1]]))
    for f, h in [(0, 0), (5, 3), (F - 1, H - 1)]:
        ref = refbank_attention(q, segs, H, frames=[f], head_list=[h], rows=rows)[(f, h)]
        assert_attn_close(got[f][rows][:, h * d:(h + 1) * d], ref, f"expr L={L} f={f} h={h}")


def test_prepared_call_matches_direct_call(B):
    """PreparedAttn (the arguments marshalled once, as the bench's round loop calls
    the library) gives the same bits as refbank_attn, and the oracle's values."""
    say("attn prepared call")
    rng = np.random.default_rng(77)
    F, L, H, d = 2, 192, 2, 40
    C = H * d
    q = rand16(rng, F, L, C)
    segs = [(rand16(rng, F, L, C), rand16(rng, F, L, C), False), (rand16(rng, 128, C), rand16(rng, 128, C), True)]
    dq = dev(q)
    dsegs = [(dev(k), dev(v)) for k, v, _ in segs]
    direct = B.refbank_attn(dq, dsegs, H)
    out = torch.empty_like(dq)
    call = B.PreparedAttn(dq, dsegs, H, out)
    for _ in range(3):  # repeated launches write the same result
        call()
    torch.cuda.synchronize()
    assert torch.equal(out, direct)
    assert_attn_close(out.cpu().numpy(), refbank_attention(q, segs, H), "prepared")
