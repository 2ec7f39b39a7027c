"""GPU parity of pl_refbank_attn_noalloc, the attention call that allocates
nothing (its key-split partials live in a scratch array the library holds on
each GPU), against pl_refbank_attn with a caller workspace: two calls in a
row, the second smaller, both launches splitting their key axis."""

import ctypes

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


def _call(B, fn, q, segs_dev, H, out, ws=None):
    F, L, C = q.shape
    d = C // H
    table, _keep = B.make_segments(segs_dev, F, C)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [ctypes.c_void_p(q.data_ptr()), q.stride(1), q.stride(0), ctypes.c_void_p(out.data_ptr()), out.stride(1),
            out.stride(0), F, L, H, d, table, len(segs_dev), float(d ** -0.5)]
    if fn == "noalloc":
        st = B.pl_refbank_attn_noalloc(*args, stream)
    else:
        st = B.pl_refbank_attn(*args, ctypes.c_void_p(ws.data_ptr()), ws.numel(), stream)
    assert st == B.PL_OK, B.last_error()


@pytest.mark.parametrize("F,L", [(2, 256), (1, 256)])  # the second call is smaller
def test_noalloc_matches_workspace_call(B, F, L):
    say("noalloc attention F =", F, "L =", L)
    lay = inputs.attention_layer(70 + F, F, L, 1280, 3)
    segs = [(lay["k_self"], lay["v_self"], False)] + [(k, v, True) for k, v in zip(lay["bank_k"], lay["bank_v"])]
    n = B.workspace_size(F, L, 8, 160, [L] * 5)
    assert n > 0, "the launch must split its key axis (so the scratch is used)"
    q = dev(lay["q"])
    segs_dev = [(dev(k), dev(v)) for k, v, _ in segs]
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    want = torch.empty_like(q)
    got = torch.full_like(q, float("nan"))
    _call(B, "workspace", q, segs_dev, 8, want, ws)
    _call(B, "noalloc", q, segs_dev, 8, got)
    torch.cuda.synchronize()
    # the same kernels, split plan and arithmetic: the same bits
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    assert_attn_close(got.cpu().numpy(), refbank_attention(lay["q"], segs, 8), "noalloc")
