"""GPU parity of the round whose pile state lives on the device
(pl_pyramid_ddim_step_device), eagerly and replayed from one captured graph.

PersonaLive write-up, section TensorRT 融合: bind() keeps the rolling latents
and the pile's bookkeeping on the device so a round is one host call.  Here
the state machine runs in the kernels; over several rounds its outputs and its
state must equal the host state machine driving pl_pyramid_ddim_step_roll,
and the oracle.  Graph replays are interleaved with eager work and each replay
is checked (memory-clearing nodes have misbehaved on replay on this platform;
the round records none).
"""

import numpy as np
import pytest

from oracle import PyramidPile, motion_bank_min_l2, pyramid_ddim_step, window_noise
from streaming_diffusion_portrait_amd import inputs
from _helpers import DDIM_REL, maxnorm_rel, say

# errors compound over a window's four steps (|A| up to 4.75 at t = 999)
CHAIN_REL = 4 * DDIM_REL * 4.75 * 2.26 * 1.37

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SEED = 9


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from streaming_diffusion_portrait_amd import binding
    binding.load()
    return binding


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _eps(r, shape):
    # a fresh epsilon estimate per round (the denoiser's output)
    return inputs.normal(1000 + r, 1, 0, shape)


def _oracle_rounds(x_t0, shape, rounds, prefill=True):
    """x_prev / x0 per round from the oracle, the pile as host integers."""
    pile = PyramidPile(prefill=prefill)
    slots = {}  # window id -> slot (the ring the library keeps)
    W = 4
    if prefill:
        for s, (wid, _) in enumerate(pile.windows):
            slots[wid] = s
    head = 0
    x = x_t0.reshape(W, -1).astype(np.float64).copy()
    out = []
    for r in range(rounds):
        evaluated, emitted = pile.round()
        new_id = evaluated[-1][0]
        slots[new_id] = (head + len(evaluated) - 1) % W
        t_slot = [999] * W
        for wid, t in evaluated:
            t_slot[slots[wid]] = t
        emit = slots[emitted] if emitted is not None else -1
        eps = _eps(r, shape).reshape(W, -1)
        xp, x0 = pyramid_ddim_step(x, eps, t_slot, emit_window=None if emit < 0 else emit)
        xp = xp.reshape(W, -1)
        if emit >= 0:
            xp[emit] = window_noise(SEED, pile.next_id, xp.shape[1])  # the next round's window
            head = (head + 1) % W
        out.append((xp.copy(), None if x0 is None else x0.reshape(-1).copy(), emit))
        x = xp
    return out, pile


@pytest.mark.parametrize("prefill", [True, False])
def test_device_state_rounds_match_host_state_and_oracle(B, prefill):
    say("device-state rounds, prefill", prefill)
    shape = (16, 4, 16, 16)
    x_np = inputs.normal(SEED, 1, 0, shape)
    rounds = 7
    ref, ref_pile = _oracle_rounds(x_np, shape, rounds, prefill)
    # device state machine, in place
    dp = B.DevicePile(4, 333, prefill=prefill)
    xd = dev(x_np)
    x0d = torch.zeros(shape[0] // 4 * int(np.prod(shape[1:])), dtype=torch.float32, device="cuda")
    # host state machine driving the rolling step, in place
    hp = B.Pile(4, 333, prefill=prefill)
    xh = dev(x_np)
    x0h = torch.zeros_like(x0d)
    for r in range(rounds):
        eps = dev(_eps(r, shape))
        dp.step(xd, eps, xd, x0d, SEED)
        _, t_slot, emit = hp.begin_round()
        B.pyramid_ddim_step(xh, eps, t_slot, x_prev=xh, x0_out=x0h if emit >= 0 else None, emit_window=emit,
                            roll=(SEED, hp._p.next_id))
        hp.end_round()
        got = xd.cpu().numpy().reshape(4, -1)
        xp_ref, x0_ref, emit_ref = ref[r]
        assert emit == emit_ref
        assert maxnorm_rel(got, xp_ref) <= CHAIN_REL, r
        assert np.allclose(got, xh.cpu().numpy().reshape(4, -1), rtol=1e-6, atol=1e-6), r
        if emit_ref >= 0:
            assert maxnorm_rel(x0d.cpu().numpy(), x0_ref) <= CHAIN_REL, r
            assert np.allclose(x0d.cpu().numpy(), x0h.cpu().numpy(), rtol=1e-6, atol=1e-6), r
        st = dp.state()
        assert (st.head, st.count, st.next_id, st.in_round) == (hp._p.head, hp._p.count, hp._p.next_id, 0)
        assert list(st.t) == list(hp._p.t) and list(st.id) == list(hp._p.id)
    assert dp.state().next_id == ref_pile.next_id


def test_captured_round_replays(B):
    """A round of the device-state step plus the motion check and one attention
    layer, captured once and replayed several times with eager work between the
    replays: every replay equals the same round run eagerly."""
    say("captured round replays")
    shape = (16, 4, 16, 16)
    x_np = inputs.normal(SEED + 1, 1, 0, shape)
    eps_np = inputs.normal(SEED + 2, 1, 0, shape)
    lay = inputs.attention_layer(SEED, 4, 256, 320, 1)
    bank_np, q_np, _ = inputs.motion_bank(SEED, 2, 512, nq=4)

    def make():
        t = dict(x=dev(x_np), eps=dev(eps_np), q=dev(lay["q"]), k=dev(lay["k_self"]), v=dev(lay["v_self"]),
                 bk=dev(lay["bank_k"][0]), bv=dev(lay["bank_v"][0]), mb=dev(bank_np), mq=dev(q_np))
        t["x0"] = torch.zeros(int(np.prod(shape)) // 4, device="cuda")
        t["o"] = torch.empty_like(t["q"])
        t["md"] = (torch.empty(4, device="cuda"), torch.empty(4, dtype=torch.int32, device="cuda"),
                   torch.empty(4, dtype=torch.uint8, device="cuda"))
        t["pile"] = B.DevicePile(4, 333)
        t["attn"] = B.PreparedAttn(t["q"], [(t["k"], t["v"]), (t["bk"], t["bv"])], 8, t["o"])
        return t

    def round_(t, stream=None):
        t["attn"](stream)
        t["pile"].step(t["x"], t["eps"], t["x"], t["x0"], SEED, stream=stream)
        B.motion_bank_min_l2(t["mq"], t["mb"], 17.0, out=t["md"], stream=stream)

    eager, graphed, warm = make(), make(), make()
    round_(warm)  # every kernel has run once before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        round_(graphed, torch.cuda.current_stream())
    torch.cuda.synchronize()
    # capturing ran nothing: the graphed buffers still hold the inputs
    assert np.array_equal(graphed["x"].cpu().numpy(), x_np)
    for r in range(5):
        round_(eager)
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        del junk
        for key in ("x", "x0", "o"):
            assert torch.equal(eager[key], graphed[key]), (r, key)
        for a, b in zip(eager["md"], graphed["md"]):
            assert torch.equal(a, b), r
        assert bytes(eager["pile"].state()) == bytes(graphed["pile"].state()), r
    # and the replayed motion check is right
    rd, ra, rf = motion_bank_min_l2(q_np, bank_np, 17.0)
    assert np.array_equal(graphed["md"][1].cpu().numpy(), ra)
