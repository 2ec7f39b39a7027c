"""GPU parity of a whole pyramid round at each anchor count m = 0..3.

The round is the one the benchmark times (PersonaLive write-up, sections
流式金字塔去噪 and 抗身份漂移的补丁: one 16-frame forward over the pile's four
windows, each attention layer's keys = its own tokens + the reference entry
+ m anchors, then the rolling DDIM step and the drift check): the 16 SD1.5
attention layers launched back to back through the same prepared calls, on
fresh seeded tensors per layer; the rolling DDIM step on the 16x4x64x64 pile
with the leaving window's x0 and the next window's noise; the motion-bank
check against 1 + m entries.  Each layer is compared with the fp64 oracle on
sampled (frame, head, row) triples; DDIM and the motion check are compared
in full.
"""

import numpy as np
import pytest

from oracle import motion_bank_min_l2, pyramid_ddim_step, refbank_attention, window_noise
from streaming_diffusion_portrait_amd import inputs
from _helpers import DDIM_REL, assert_attn_close, maxnorm_rel, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SEED = 4  # the benchmark's round seed: at m = 3 these are its inputs exactly
F, H = 16, 8


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_diffusion_portrait_amd import binding
    binding.load()
    return binding


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("m", [0, 1, 2, 3])
def test_full_round(B, m):
    say("round m =", m, "inputs")
    layers = []
    for li, (name, L, C) in enumerate(inputs.SD15_LAYERS):
        lay = inputs.attention_layer(1000 * SEED + li, F, L, C, m)
        q = dev(lay["q"])
        segs = [(dev(lay["k_self"]), dev(lay["v_self"]))]
        segs += [(dev(k), dev(v)) for k, v in zip(lay["bank_k"], lay["bank_v"])]
        out = torch.empty_like(q)
        layers.append((name, L, C, lay, out, B.PreparedAttn(q, segs, H, out), (q, segs)))
    x_t_np, eps_np = inputs.ddim_pile(SEED, (16, 4, 64, 64))
    x_t, eps = dev(x_t_np), dev(eps_np)
    x_prev = torch.empty_like(x_t)
    x0 = torch.empty((4, 4, 64, 64), dtype=torch.float32, device="cuda")
    bank_np, q_np, _ = inputs.motion_bank(SEED + m, 1 + m, 512, nq=64)
    mb, mq = dev(bank_np), dev(q_np)
    torch.cuda.synchronize()

    say("round m =", m, "launch")
    for *_, call, _keep in layers:
        call()
    pile = B.Pile(4, 333)
    _, t_slot, emit = pile.begin_round()
    B.pyramid_ddim_step(x_t, eps, t_slot, x_prev=x_prev, x0_out=x0, emit_window=emit, roll=(SEED, 4))
    pile.end_round()
    md, am, ex = B.motion_bank_min_l2(mq, mb, 17.0)
    torch.cuda.synchronize()

    rng = np.random.default_rng(100 + m)
    for name, L, C, lay, out, _call, _keep in layers:
        say("round m =", m, "layer", name)
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got)), name
        d = C // H
        segs = [(lay["k_self"], lay["v_self"], False)]
        segs += [(k, v, True) for k, v in zip(lay["bank_k"], lay["bank_v"])]
        for f, h in {(0, 0), (F - 1, H - 1), (int(rng.integers(F)), int(rng.integers(H)))}:
            rows = np.unique(np.concatenate([rng.choice(L, size=min(24, L), replace=False), [0, L - 1]]))
            ref = refbank_attention(lay["q"], segs, H, frames=[f], head_list=[h], rows=rows)[(f, h)]
            assert_attn_close(got[f][rows][:, h * d:(h + 1) * d], ref, f"m={m} {name} f={f} h={h}")

    say("round m =", m, "ddim + motion")
    assert t_slot == [0, 333, 666, 999] and emit == 0
    ref_prev, ref_x0 = pyramid_ddim_step(x_t_np, eps_np, t_slot, emit_window=emit)
    ref_prev = ref_prev.reshape(4, -1)
    ref_prev[emit] = window_noise(SEED, 4, ref_prev.shape[1])
    assert maxnorm_rel(x_prev.cpu().numpy().reshape(4, -1), ref_prev) <= DDIM_REL
    assert maxnorm_rel(x0.cpu().numpy().reshape(ref_x0.shape), ref_x0) <= DDIM_REL
    rd, ra, rf = motion_bank_min_l2(q_np, bank_np, 17.0)
    md, am, ex = md.cpu().numpy(), am.cpu().numpy(), ex.cpu().numpy()
    keep = np.abs(rd - 17.0) > 1e-9
    assert np.array_equal(ex[keep].astype(bool), rf[keep])
    assert np.array_equal(am, ra)
    assert np.max(np.abs(md - rd) / rd) <= 1e-6
