"""Attention cases run against the bounds-checking build (not collected by
pytest: tests/test_gpu_debug_bounds.py runs this file in a child process whose
PL_LIBRARY names libpl_dbg.so).  Every path of the attention kernels --
pipelined and tile-by-tile key sequences, ragged tails, every head dim, the
key split and its merge, frames of at most 64 rows (two waves per query
block), block-causal chunks, short contexts, strided views, the call without a
workspace -- is run and compared with the oracle; the line printed last is
JSON with the access-violation mask and the worst errors."""

import ctypes
import json
import os
import sys
import zlib

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

from oracle import chunk_causal_attention, refbank_attention  # noqa: E402
from streaming_diffusion_portrait_amd import binding as B  # noqa: E402
from _helpers import attn_errors  # noqa: E402


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rand16(rng, *shape):
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def case_segments(name, d, F, L, H, segspec):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    C = H * d
    q = rand16(rng, F, L, C)
    segs = []
    for ln, shared in segspec:
        shape = (ln, C) if shared else (F, ln, C)
        segs.append((rand16(rng, *shape), rand16(rng, *shape), shared))
    return q, segs


def main():
    B.load()
    if B.debug_bounds(reset=True) is None:
        print(json.dumps({"error": "the loaded library has no bounds checks: " + B.LIB_PATH}))
        return 2
    results = []

    def record(name, got, ref):
        e = attn_errors(got, ref)
        e["name"] = name
        results.append(e)
        print(json.dumps(e), flush=True)

    cases = [
        ("d32 ragged", 32, 2, 257, 2, [(257, False), (256, True), (5, True)]),
        ("d40 ragged", 40, 3, 300, 2, [(300, False), (100, True), (37, True)]),
        ("d40 whole tiles", 40, 2, 256, 2, [(256, False), (512, True), (64, True)]),
        ("d80 ragged", 80, 2, 130, 2, [(130, False), (64, True), (65, True), (1, True)]),
        ("d80 whole tiles", 80, 2, 256, 1, [(256, False), (64, True), (192, True)]),
        ("d160 ragged", 160, 2, 70, 2, [(70, False), (33, True)]),
        ("d160 small frame", 160, 3, 37, 2, [(37, False), (100, True), (1, True)]),
        ("one-frame key split 16^2", 160, 1, 256, 8, [(256, False)] + [(256, True)] * 4),
        ("short context d40", 40, 2, 200, 2, [(32, True)]),
        ("short context d80", 80, 2, 130, 2, [(50, False)]),
        ("short context d160", 160, 2, 70, 1, [(1, True)]),
    ]
    for name, d, F, L, H, spec in cases:
        q, segs = case_segments(name, d, F, L, H, spec)
        out = B.refbank_attn(dev(q), [(dev(k), dev(v)) for k, v, _ in segs], H)
        torch.cuda.synchronize()
        record(name, out.cpu().numpy(), refbank_attention(q, segs, H))

    # strided views of one fused [q | k | v] buffer, output into a padded buffer
    rng = np.random.default_rng(11)
    F, L, H, d = 2, 200, 2, 40
    C = H * d
    qkv = rand16(rng, F, L, 3 * C)
    dq = dev(qkv)
    out = torch.zeros(F, L + 3, C + 8, dtype=torch.float16, device="cuda")[:, :L, :C]
    B.refbank_attn(dq[..., :C], [(dq[..., C:2 * C], dq[..., 2 * C:])], H, out=out)
    torch.cuda.synchronize()
    record("strided views", out.cpu().numpy(),
           refbank_attention(qkv[..., :C], [(qkv[..., C:2 * C], qkv[..., 2 * C:], False)], H))

    # the call without a workspace (partials in the library's scratch), splitting
    q, segs = case_segments("noalloc split", 160, 1, 64, 8, [(64, False)] + [(512, True)] * 4)
    dsegs = [(dev(k), dev(v)) for k, v, _ in segs]
    dqn = dev(q)
    outn = torch.empty_like(dqn)
    table, _keep = B.make_segments(dsegs, 1, q.shape[2])
    st = B.pl_refbank_attn_noalloc(ctypes.c_void_p(dqn.data_ptr()), dqn.stride(1), dqn.stride(0),
                                   ctypes.c_void_p(outn.data_ptr()), outn.stride(1), outn.stride(0), 1, 64, 8, 160,
                                   table, len(dsegs), float(160 ** -0.5),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, B.last_error()
    torch.cuda.synchronize()
    record("noalloc split", outn.cpu().numpy(), refbank_attention(q, segs, 8))

    # block-causal chunks
    rng = np.random.default_rng(13)
    F, L, H, d = 2, 150, 2, 40
    C = H * d
    q = rand16(rng, F, L, C)
    ks, vs = rand16(rng, F, L, C), rand16(rng, F, L, C)
    kb, vb = rand16(rng, 70, C), rand16(rng, 70, C)
    out = B.chunked_attn(dev(q), (dev(ks), dev(vs)), [(dev(kb), dev(vb))], H, chunk_len=40, max_history=1)
    torch.cuda.synchronize()
    record("block-causal chunks", out.cpu().numpy(),
           chunk_causal_attention(q, (ks, vs), [(kb, vb)], H, chunk_len=40, max_history=1))

    mask = B.debug_bounds(reset=True)
    print(json.dumps({"mask": mask, "cases": len(results),
                      "max_abs": max(r["max_abs"] for r in results),
                      "mean_abs": max(r["mean_abs"] for r in results)}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
