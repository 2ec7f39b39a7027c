"""The attention kernels' indexing under the bounds-checking build.

libpl_dbg.so (built by ``__graft_entry__.build()`` next to libpl.so, or
``python -m streaming_diffusion_portrait_amd.build --debug-bounds``) checks
every global and LDS access of the attention kernels against its buffer before
making it.  tests/bounds_cases.py runs every attention path through that build
in a child process and reports the mask of access sites that failed their
check: it must be empty, and the results must still match the oracle.  Also
here: two runs of the normal build give the same bits.
"""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import refbank_attention
from _helpers import ATTN_MAX_ABS, ATTN_MEAN_ABS, assert_attn_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DBG = os.path.join(ROOT, "streaming_diffusion_portrait_amd", "libpl_dbg.so")


def test_every_attention_access_stays_in_its_buffer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(DBG):
        pytest.skip("libpl_dbg.so not built (run __graft_entry__.build())")
    say("attn bounds-checking build")
    env = dict(os.environ)
    env["PL_LIBRARY"] = DBG
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "bounds_cases.py")], env=env,
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert r.returncode == 0 and lines, r.stdout[-3000:] + r.stderr[-3000:]
    last = json.loads(lines[-1])
    assert last["mask"] == 0, f"access sites out of bounds: mask {last['mask']:#x}"
    assert last["cases"] >= 14, last
    assert last["max_abs"] <= ATTN_MAX_ABS and last["mean_abs"] <= ATTN_MEAN_ABS, last


def test_runs_are_bitwise_identical():
    """Two runs of the same calls give the same bits (no atomics, fixed merge
    order): a pipelined 64^2-shaped layer slice and a key-split launch."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_diffusion_portrait_amd import binding as B
    B.load()
    say("attn determinism")
    rng = np.random.default_rng(21)
    for F, L, H, d, spec in [(2, 512, 8, 40, [(512, False), (512, True), (512, True)]),
                             (1, 256, 8, 160, [(256, False)] + [(256, True)] * 4)]:
        C = H * d
        q = rng.standard_normal((F, L, C), dtype=np.float32).astype(np.float16)
        segs = []
        for ln, shared in spec:
            shape = (ln, C) if shared else (F, ln, C)
            segs.append((rng.standard_normal(shape, dtype=np.float32).astype(np.float16),
                         rng.standard_normal(shape, dtype=np.float32).astype(np.float16), shared))
        dq = torch.from_numpy(q).cuda()
        dsegs = [(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()) for k, v, _ in segs]
        a = B.refbank_attn(dq, dsegs, H)
        b = B.refbank_attn(dq, dsegs, H)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert_attn_close(a.cpu().numpy(), refbank_attention(q, segs, H), "determinism case")
