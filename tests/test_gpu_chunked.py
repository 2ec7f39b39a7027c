"""GPU parity of block-causal attention over chunked sequences
(pl_refbank_attn_chunked) against the fp64 oracle.

LPM write-up, section 6.3 分块因果注意力, and the deep-compression-VAE
write-up: full attention inside a chunk, earlier chunks only across (a
limited number of them), plus persistent reference tokens.  Cases: chunk
lengths that do and do not divide the sequence, history limits, one chunk
(plain attention), one-row chunks, every head dim.
"""

import zlib

import numpy as np
import pytest

from oracle import chunk_causal_attention
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


CASES = [
    # (name, d, F, L, H, chunk_len, max_history, shared lens)
    ("d40 4 chunks, all history", 40, 2, 256, 2, 64, -1, [64]),
    ("d40 ragged last chunk, one earlier chunk", 40, 2, 300, 2, 128, 1, [64, 7]),
    ("d40 one chunk = plain attention", 40, 1, 200, 2, 200, -1, [64]),
    ("d80 chunks of 96 rows, two earlier", 80, 2, 400, 1, 96, 2, [33]),
    ("d160 no reference tokens", 160, 1, 130, 1, 64, -1, []),
    ("d32 one-row chunks, no history", 32, 1, 70, 2, 1, 0, [5]),
]


@pytest.mark.parametrize("name,d,F,L,H,cl,hist,shared_lens", CASES, ids=[c[0] for c in CASES])
def test_chunked_matches_oracle(B, name, d, F, L, H, cl, hist, shared_lens):
    say("chunked", name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    C = H * d
    r = lambda *s: rng.standard_normal(s, dtype=np.float32).astype(np.float16)
    q, k, v = r(F, L, C), r(F, L, C), r(F, L, C)
    shared = [(r(n, C), r(n, C)) for n in shared_lens]
    out = B.chunked_attn(dev(q), (dev(k), dev(v)), [(dev(a), dev(b)) for a, b in shared], H, cl, hist)
    torch.cuda.synchronize()
    ref = chunk_causal_attention(q, (k, v), shared, H, cl, hist)
    assert_attn_close(out.cpu().numpy(), ref, name)
