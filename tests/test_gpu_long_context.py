"""GPU parity for long key sequences, against the fp64 oracle (whole outputs).

A reference bank can hold far more entries than the round's 1 + 3: the key
axis of one call may reach 2^24 keys.  These cases run one frame against

* a bank of 2^20 + 13 keys at d = 40 (some 16,400 key tiles through the
  pipelined loop, a ragged last tile);
* a bank of 2^17 + 13 keys whose rows sit 32 KB apart (columns of a wider
  buffer), so its K and V each span 4.3 GB and the segment offsets the kernel
  walks pass 2^31 and 2^32 bytes;
* a bank of 300,007 keys at d = 160 on a frame of 40 rows (two waves per query
  block; the one-frame launch splits the key axis into about 250 parts and
  merges them).
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


CASES = [
    # (name, d, H, Lq, bank length, bank row pitch in elements or None)
    ("d40 bank of 2^20 + 13 keys", 40, 2, 77, (1 << 20) + 13, None),
    ("d40 bank of 2^17 + 13 keys, 32 KB row pitch", 40, 2, 50, (1 << 17) + 13, 16384),
    ("d160 small frame, bank of 300007 keys", 160, 1, 40, 300007, None),
]


@pytest.mark.parametrize("name,d,H,L,nbank,pitch", CASES, ids=[c[0] for c in CASES])
def test_long_bank_full_compare(B, name, d, H, L, nbank, pitch):
    say("attn long", name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    C = H * d
    q = rng.standard_normal((1, L, C), dtype=np.float32).astype(np.float16)
    k_self = rng.standard_normal((1, L, C), dtype=np.float32).astype(np.float16)
    v_self = rng.standard_normal((1, L, C), dtype=np.float32).astype(np.float16)
    k_bank = rng.standard_normal((nbank, C), dtype=np.float32).astype(np.float16)
    v_bank = rng.standard_normal((nbank, C), dtype=np.float32).astype(np.float16)
    if pitch is None:
        dk, dv = dev(k_bank), dev(v_bank)
    else:
        kbuf = torch.zeros((nbank, pitch), dtype=torch.float16, device="cuda")
        vbuf = torch.zeros((nbank, pitch), dtype=torch.float16, device="cuda")
        dk, dv = kbuf[:, :C], vbuf[:, :C]
        dk.copy_(dev(k_bank))
        dv.copy_(dev(v_bank))
        assert dk.stride(0) * 2 * nbank > (1 << 32)
    if d == 160:
        assert B.workspace_size(1, L, H, d, [L, nbank]) > 0, "the one-frame launch must split its key axis"
    out = B.refbank_attn(dev(q), [(dev(k_self), dev(v_self)), (dk, dv)], H)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = refbank_attention(q, [(k_self, v_self, False), (k_bank, v_bank, True)], H)
    e = assert_attn_close(got, ref, name)
    assert e["norm_rel"] <= 2e-3, e
