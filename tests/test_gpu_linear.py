"""GPU parity of pl_linear (the projections either side of the attention)
against the fp64 oracle, and a projection -> attention chain on strided views."""

import zlib

import numpy as np
import pytest

from oracle import linear, refbank_attention
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


def case(name, M, N, K, bias):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    x = rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)
    w = (rng.standard_normal((N, K), dtype=np.float32) / np.sqrt(K)).astype(np.float16)
    b = rng.standard_normal(N, dtype=np.float32) if bias else None
    return x, w, b


def check(got, ref, K):
    # fp16 output: rounding to nearest (2^-11 relative) plus the fp32 sum over K terms
    got = np.asarray(got, dtype=np.float64)
    tol = np.abs(ref) * 2.0 ** -11 + 2e-6 * np.sqrt(K) * (1.0 + np.abs(ref))
    assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) - tol))


SMALL = [("ragged rows", 300, 128, 48, True), ("one row", 1, 64, 16, False), ("clip kv", 1, 640, 768, False),
         ("expression kv", 32 * 16, 640, 16, False), ("wide", 77, 1280, 1280, True), ("many tiles", 1000, 192, 320, False),
         # 84 tiles of 128 x 64 (not a multiple of the 8 XCDs), grouped 2 row tiles high
         ("odd tile count", 1500, 448, 256, True)]


@pytest.mark.parametrize("name,M,N,K,bias", SMALL, ids=[c[0] for c in SMALL])
def test_linear_full_compare(B, name, M, N, K, bias):
    say("linear", name, M, N, K)
    x, w, b = case(name, M, N, K, bias)
    got = B.linear(dev(x), dev(w), dev(b) if bias else None)
    torch.cuda.synchronize()
    check(got.cpu().numpy(), linear(x, w, b), K)


# Shapes that select each tile configuration of the K % 64 == 0 kernel
# (128 x 64, 256 x 64 for large M, 128 x 192 for large M with N a multiple of
# 192, 256 x 256 for long K, 128 x 128 with three stages for long K and few
# rows), with ragged row tails.
TILES = [("128x64 tiles", 333, 128, 128), ("256x64 tiles", 16300, 1024, 128), ("128x192 tiles", 16300, 1920, 640),
         ("256x256 tiles", 3600, 3840, 1024), ("128x128 3-stage tiles", 1000, 3840, 1024)]


@pytest.mark.parametrize("row_stores", [True, False], ids=["row stores", "direct stores"])
@pytest.mark.parametrize("name,M,N,K", TILES, ids=[c[0] for c in TILES])
def test_tile_configs_sampled(B, name, M, N, K, row_stores):
    """Every tile configuration, with bias, through both output paths: y 16-byte
    aligned with a row pitch of 8 elements (tile staged in LDS, whole 16-byte row
    chunks stored) and a pitch of N + 4 (8-byte stores straight from registers)."""
    say("linear tiles", name, M, N, K, "row" if row_stores else "direct")
    x, w, b = case(name, M, N, K, True)
    if row_stores:
        out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    else:
        out = torch.empty((M, N + 4), dtype=torch.float16, device="cuda")[:, :N]
    got = B.linear(dev(x), dev(w), dev(b), out=out)
    torch.cuda.synchronize()
    # rows around the 128- and 256-row tile edges near both ends, plus a random spread
    edges = [r for t in (128, 256, 512, (M // 128) * 128, (M // 256) * 256) for r in (t - 1, t) if r < M]
    rows = np.unique(np.concatenate([np.random.default_rng(M).integers(0, M, 200), [0, M - 1], edges]))
    check(got.cpu().numpy()[rows], linear(x[rows], w, b), K)


@pytest.mark.parametrize("L,C", [(4096, 320), (1024, 640), (256, 1280), (64, 1280)])
def test_fused_qkv_projection_sampled(B, L, C):
    """to_q / to_k / to_v as one [3C, C] weight over the 16 frames of a level."""
    say("linear qkv", L, C)
    F = 16
    x, w, _ = case(f"qkv{L}", F * L, 3 * C, C, False)
    got = B.linear(dev(x), dev(w))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(L).integers(0, F * L, 256), [0, F * L - 1]]))
    check(got.cpu().numpy()[rows], linear(x[rows], w), C)


def test_projection_then_attention_on_strided_views(B):
    """x -> [q | k | v] with one fused weight, the bank's k | v with another, then the
    attention reads q, k, v as column slices (row stride 3C) -- no copies."""
    say("linear -> attention chain")
    F, L, C, H = 2, 200, 128, 4  # d = 32; 3C and 2C multiples of 64
    rng = np.random.default_rng(5)
    x = rng.standard_normal((F, L, C), dtype=np.float32).astype(np.float16)
    hb = rng.standard_normal((L, C), dtype=np.float32).astype(np.float16)  # bank hidden states
    wqkv = (rng.standard_normal((3 * C, C), dtype=np.float32) / np.sqrt(C)).astype(np.float16)
    wkv = wqkv[C:]
    y = B.linear(dev(x), dev(wqkv))              # [F, L, 3C]
    ybank = B.linear(dev(hb), dev(np.ascontiguousarray(wkv)))  # [L, 2C]
    q, k, v = y[..., :C], y[..., C:2 * C], y[..., 2 * C:]
    kb, vb = ybank[:, :C], ybank[:, C:]
    out = B.refbank_attn(q, [(k, v), (kb, vb)], H)
    torch.cuda.synchronize()
    # oracle: the same chain in fp64, with the projections rounded to fp16 as the kernel's inputs are
    yr = linear(x.reshape(-1, C), wqkv).reshape(F, L, 3 * C)
    ybr = linear(hb, wkv)
    assert np.allclose(y.cpu().numpy(), yr, atol=4e-3, rtol=2e-3)
    y16 = y.cpu().numpy()
    yb16 = ybank.cpu().numpy()
    segs = [(y16[..., C:2 * C], y16[..., 2 * C:], False), (yb16[:, :C], yb16[:, C:], True)]
    ref = refbank_attention(y16[..., :C], segs, H)
    assert_attn_close(out.cpu().numpy(), ref, "chain")
    assert np.allclose(yb16, ybr, atol=4e-3, rtol=2e-3)


@pytest.mark.parametrize("col0", [8, 4], ids=["row stores", "direct stores"])
@pytest.mark.parametrize("M,N,K", [(700, 192, 320), (16400, 1024, 128), (26300, 960, 320)],
                         ids=["128x64 tiles", "256x64 tiles", "128x192 tiles"])
def test_strided_views(B, M, N, K, col0):
    """x a column slice of a wider buffer (row pitch K + 64), y written into a
    padded buffer at column col0 (16-byte aligned rows: LDS-staged stores; 8-byte:
    direct stores); nothing outside y's view changes."""
    say("linear strided", M, N, K, col0)
    x, w, b = case(f"strided{M}", M, N, K, True)
    xbuf = torch.zeros(M, K + 64, dtype=torch.float16, device="cuda")
    xbuf[:, 32:32 + K] = dev(x)
    xv = xbuf[:, 32:32 + K]
    ybuf = torch.full((M + 2, N + 16), -7.0, dtype=torch.float16, device="cuda")
    yv = ybuf[1:M + 1, col0:col0 + N]
    B.linear(xv, dev(w), dev(b), out=yv)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(3).integers(0, M, 200), [0, M - 1]]))
    check(yv.cpu().numpy()[rows], linear(x[rows], w, b), K)
    rest = ybuf.cpu().numpy().copy()
    rest[1:M + 1, col0:col0 + N] = -7.0
    assert (rest == np.float16(-7.0)).all()
