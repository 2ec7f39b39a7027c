"""GPU parity of pl_pyramid_ddim_step and pl_motion_bank_min_l2 against the oracle."""

import numpy as np
import pytest

from oracle import pyramid_ddim_step, sd_scaled_linear_alphas_cumprod, motion_bank_min_l2
from streaming_diffusion_portrait_amd import inputs
from _helpers import DDIM_REL, maxnorm_rel, say

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


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _ddim_case(B, shape, ts, emit, seed, inplace=False, ab=None, fin=-1.0):
    x_t, eps = inputs.ddim_pile(seed, shape)
    dx, de = dev(x_t), dev(eps)
    out = dx if inplace else None
    xp, x0 = B.pyramid_ddim_step(dx, de, ts, x_prev=out, emit_window=emit, alphas_cumprod=ab,
                                 final_alpha_cumprod=fin)
    ab_ref = sd_scaled_linear_alphas_cumprod() if ab is None else np.asarray(ab)
    ref_prev, ref_x0 = pyramid_ddim_step(x_t, eps, ts, 333, ab_ref,
                                         None if fin < 0 else fin, emit_window=None if emit < 0 else emit)
    got_prev = host(xp)
    r1 = maxnorm_rel(got_prev, ref_prev)
    assert r1 <= DDIM_REL, r1
    if emit >= 0:
        W = len(ts)
        r2 = maxnorm_rel(host(x0).reshape(ref_x0.shape), ref_x0)
        assert r2 <= DDIM_REL, r2
        # the emitted window's x0 is exactly what the oracle's window-level step returns
        assert ref_x0.shape[0] * W == shape[0]
    return r1


def test_ddim_tiny(B):
    say("ddim tiny [16,4,8,8]")
    _ddim_case(B, (16, 4, 8, 8), [999, 666, 333, 0], 3, 0)


def test_ddim_full_pile_rolled_slots(B):
    say("ddim full [16,4,64,64] rolled")
    _ddim_case(B, (16, 4, 64, 64), [333, 0, 999, 666], 1, 4)


def test_ddim_in_place(B):
    say("ddim in place")
    _ddim_case(B, (16, 4, 64, 64), [999, 666, 333, 0], 3, 5, inplace=True)


def test_ddim_no_emit_and_custom_schedule(B):
    say("ddim custom schedule")
    ab = np.linspace(0.999, 0.01, 1000)
    _ddim_case(B, (16, 4, 8, 8), [999, 666, 333, 0], -1, 6, ab=ab)
    _ddim_case(B, (16, 4, 8, 8), [999, 666, 333, 0], 3, 7, ab=ab, fin=1.0)


def test_ddim_scalar_path_odd_sizes(B):
    say("ddim scalar path")
    _ddim_case(B, (8, 3, 5, 7), [999, 666, 333, 0], 0, 8)


def test_ddim_misaligned_pointer(B):
    say("ddim misaligned")
    x_t, eps = inputs.ddim_pile(9, (4 * 257,))
    buf = torch.zeros(4 * 257 + 1, dtype=torch.float32, device="cuda")
    dx = buf[1:]
    dx.copy_(torch.from_numpy(x_t))
    xp, x0 = B.pyramid_ddim_step(dx, dev(eps), [999, 666, 333, 0], emit_window=3)
    ref_prev, ref_x0 = pyramid_ddim_step(x_t, eps, [999, 666, 333, 0], emit_window=3)
    assert maxnorm_rel(host(xp), ref_prev) <= DDIM_REL
    assert maxnorm_rel(host(x0), ref_x0) <= DDIM_REL


def test_ddim_large_sweep_size(B):
    say("ddim 4 x 2^22")
    _ddim_case(B, (4, 1 << 22), [999, 666, 333, 0], 3, 10)


def test_ddim_recovers_x0_from_forward_marginal(B):
    # x_t built from known (x0, eps) at each window's t: the emitted x0 and every
    # x_prev land where the forward process puts them
    say("ddim closed form on GPU")
    ab = sd_scaled_linear_alphas_cumprod()
    ts = [999, 666, 333, 0]
    x0 = inputs.normal(12, 2, 0, (16, 4, 64, 64)).astype(np.float64)
    eps = inputs.normal(12, 2, 1, (16, 4, 64, 64)).astype(np.float64)
    x_t = np.empty_like(x0)
    for w, t in enumerate(ts):
        blk = slice(4 * w, 4 * w + 4)
        x_t[blk] = np.sqrt(ab[t]) * x0[blk] + np.sqrt(1 - ab[t]) * eps[blk]
    x_t32, eps32 = x_t.astype(np.float32), eps.astype(np.float32)
    xp, x0_out = B.pyramid_ddim_step(dev(x_t32), dev(eps32), ts, emit_window=3)
    ref_prev, ref_x0 = pyramid_ddim_step(x_t32, eps32, ts, emit_window=3)
    assert maxnorm_rel(host(x0_out).reshape(4, 4, 64, 64), ref_x0) <= DDIM_REL
    assert maxnorm_rel(host(xp), ref_prev) <= DDIM_REL
    # and, up to the fp32 rounding of the inputs, x0 is the one x_t was built from
    assert np.max(np.abs(host(x0_out).reshape(4, 4, 64, 64) - x0[12:16])) <= 1e-5


def _motion_check(B, bank, queries, threshold=17.0, margin=1e-9):
    md, am, ex = B.motion_bank_min_l2(dev(queries), dev(bank), threshold)
    md, am, ex = host(md), host(am), host(ex)
    rd, ra, rf = motion_bank_min_l2(queries, bank, threshold)
    keep = np.abs(rd - threshold) > margin
    assert np.array_equal(ex[keep].astype(bool), rf[keep])
    assert np.array_equal(am, ra)
    assert np.max(np.abs(md - rd) / np.maximum(rd, 1e-30)) <= 1e-5
    return keep.sum()


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_motion_random_straddling_threshold(B, n):
    say("motion n =", n)
    bank, queries, _ = inputs.motion_bank(100 + n, n, 512, nq=256)
    kept = _motion_check(B, bank, queries)
    assert kept >= 250
    _, _, flags = motion_bank_min_l2(queries, bank)
    assert 0 < flags.sum() < len(flags)  # both decisions occur


def test_motion_exact_ties_and_duplicates(B):
    say("motion ties")
    rng = np.random.default_rng(0)
    e = rng.standard_normal(512).astype(np.float32)
    bank = np.stack([e + 40, e.copy(), e.copy(), e - 40]).astype(np.float32)
    q = e[None, :].copy()
    ib = np.zeros((2, 512), dtype=np.float32)
    ib[1] = 100.0
    iq = np.zeros((3, 512), dtype=np.float32)
    iq[0, 7] = 17.0                      # exactly 17: not an exceed
    iq[1, 100], iq[1, 300] = 8.0, 15.0   # 8-15-17 triangle: exactly 17
    iq[2, 7] = 17.0 + 2.0 ** -10          # just above
    md, am, ex = [host(t) for t in B.motion_bank_min_l2(dev(iq), dev(ib), 17.0)]
    assert md[0] == 17.0 and md[1] == 17.0 and md[2] > 17.0
    assert list(ex) == [0, 0, 1] and list(am) == [0, 0, 0]
    md, am, ex = [host(t) for t in B.motion_bank_min_l2(dev(q), dev(bank), 17.0)]
    assert md[0] == 0.0 and am[0] == 1 and ex[0] == 0


def test_motion_odd_dimension(B):
    say("motion D=100")
    bank, queries, _ = inputs.motion_bank(7, 3, 100, nq=64, sigma_range=(1.2, 2.2))
    _motion_check(B, bank, queries)
