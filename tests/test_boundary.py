"""CPU tests of the C ABI: the library loads, exports every declared symbol,
rejects invalid arguments before touching the device, and its host-side pile
state machine matches the oracle's queue.

No call here reaches a kernel launch: every call has an argument that
validation rejects, and validation runs before any HIP call.  The fake device
addresses below are never dereferenced.
"""

import ctypes
import os
import re

import pytest

from streaming_diffusion_portrait_amd import binding as B
from oracle import PyramidPile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "pl.h")

A = ctypes.c_void_p(0x10000)        # fake, 16-byte aligned "device" address
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)      # fake, 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libpl.so not built")
    return B.load()


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pl_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_debug_bounds_outside_a_checking_build(lib):
    """The normal build answers the bounds report with PL_EUNSUPPORTED and a
    zero mask, before any HIP call; a NULL mask is PL_EINVAL."""
    mask = ctypes.c_uint64(123)
    assert lib.pl_debug_bounds(ctypes.byref(mask), 1) == B.PL_EUNSUPPORTED
    assert mask.value == 0
    assert "PL_DEBUG_BOUNDS" in B.last_error()
    assert lib.pl_debug_bounds(None, 0) == B.PL_EINVAL
    assert B.debug_bounds() is None


def test_version_and_status_strings(lib):
    assert lib.pl_abi_version() == 5
    assert [B.status_name(s) for s in range(4)] == ["PL_OK", "PL_EINVAL", "PL_EUNSUPPORTED", "PL_EDEVICE"]
    assert B.status_name(99) == "PL_UNKNOWN"


def _segs(*specs):
    arr = (B.pl_kv_segment * max(1, len(specs)))()
    for i, (k, v, ln, ld, fs) in enumerate(specs):
        arr[i] = B.pl_kv_segment(k, v, ln, ld, fs)
    return arr


def _attn(q=A, q_ld=64, q_fs=64 * 256, o=A2, o_ld=64, o_fs=64 * 256, F=16, L=256, H=2, d=32, segs=None, nseg=1,
          scale=0.17):
    if segs is None:
        segs = _segs((A, A2, 256, 64, 0))
    return B.pl_refbank_attn(q, q_ld, q_fs, o, o_ld, o_fs, F, L, H, d, segs, nseg, scale, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.PL_EINVAL),
    (dict(o=None), B.PL_EINVAL),
    (dict(F=0), B.PL_EINVAL),
    (dict(L=0), B.PL_EINVAL),
    (dict(H=0), B.PL_EINVAL),
    (dict(nseg=0), B.PL_EINVAL),
    (dict(nseg=9), B.PL_EINVAL),
    (dict(scale=0.0), B.PL_EINVAL),
    (dict(scale=float("nan")), B.PL_EINVAL),
    (dict(d=64, q_ld=128, o_ld=128), B.PL_EUNSUPPORTED),
    (dict(d=48, q_ld=96, o_ld=96), B.PL_EUNSUPPORTED),
    (dict(q_ld=32), B.PL_EINVAL),
    (dict(q_ld=68), B.PL_EUNSUPPORTED),
    (dict(q=MIS), B.PL_EUNSUPPORTED),
    (dict(o_fs=64 * 100), B.PL_EINVAL),
    (dict(segs=_segs((A, A2, 0, 64, 0))), B.PL_EINVAL),
    (dict(segs=_segs((None, A2, 16, 64, 0))), B.PL_EINVAL),
    (dict(segs=_segs((A, A2, 16, 48, 0))), B.PL_EINVAL),
    (dict(segs=_segs((A, A2, 16, 64, 12))), B.PL_EUNSUPPORTED),
    (dict(segs=_segs((A, MIS, 16, 64, 0))), B.PL_EUNSUPPORTED),
    (dict(segs=_segs((A, A2, 16, 64, -64))), B.PL_EINVAL),
    (dict(segs=_segs((A, A2, 1 << 24, 64, 0), (A, A2, 1, 64, 0)), nseg=2), B.PL_EINVAL),
])
def test_attention_rejects(lib, kw, status):
    assert _attn(**kw) == status
    assert B.last_error() != ""


def test_attention_second_segment_checked(lib):
    segs = _segs((A, A2, 256, 64, 0), (A, A2, 0, 64, 0))
    assert _attn(segs=segs, nseg=2) == B.PL_EINVAL
    assert "segment 1" in B.last_error()


def test_attention_rejects_output_overlap(lib):
    # o is the q buffer itself, or o sits on a segment's values
    big = _segs((ctypes.c_void_p(0x900000), ctypes.c_void_p(0xA00000), 256, 64, 0))
    assert _attn(o=A, segs=big) == B.PL_EINVAL and "o overlaps q" in B.last_error()
    assert _attn(o=ctypes.c_void_p(0xA00000 + 64 * 2 * 8), segs=big) == B.PL_EINVAL
    assert "segment 0" in B.last_error()
    assert _attn(o=ctypes.c_void_p(0xA00000), segs=big) == B.PL_EINVAL
    assert "segment 0" in B.last_error()


def test_attention_fused_column_slices(lib):
    # q | k | v | o as column slices of one [F, L, 4C] buffer (row stride 4C):
    # the views interleave in memory but share no element, so the overlap
    # check passes and the call stops at the next check (total key length)
    F, L, C = 2, 16, 64
    base = 0x400000
    ld, fs = 4 * C, 4 * C * L
    q, k, v, o = (ctypes.c_void_p(base + 2 * C * i) for i in range(4))
    too_long = _segs((k, v, (1 << 24) + 1, ld, fs))
    st = B.pl_refbank_attn(q, ld, fs, o, ld, fs, F, L, 2, 32, too_long, 1, 0.17, None, 0, None)
    assert st == B.PL_EINVAL and "total key length" in B.last_error()
    # the same buffer with o shifted half a slice into v's columns overlaps
    o_bad = ctypes.c_void_p(base + 2 * C * 2 + C)
    st = B.pl_refbank_attn(q, ld, fs, o_bad, ld, fs, F, L, 2, 32, too_long, 1, 0.17, None, 0, None)
    assert st == B.PL_EINVAL and "segment 0" in B.last_error()


def _wsize(lib, F, L, H, d, lens):
    arr = (ctypes.c_int64 * max(1, len(lens)))(*lens)
    return lib.pl_refbank_attn_workspace_size(F, L, H, d, arr, len(lens))


def test_workspace_size(lib):
    # launches that fill the CUs, or whose key axis is too short to split, need none
    assert _wsize(lib, 16, 4096, 8, 40, [4096] * 5) == 0
    assert _wsize(lib, 16, 1024, 8, 80, [1024] * 5) == 0
    assert _wsize(lib, 16, 256, 8, 160, [256] * 5) == 0
    assert _wsize(lib, 16, 64, 8, 160, [64] * 5) == 0
    # one frame of the 16^2 level with the 4x bank (20 key tiles, 16 workgroups):
    # five splits of four tiles (the split count minimises 1.3 us per tile per
    # split against each split's partials round trip); partial O, offset and
    # row sum in fp32 per (frame, head, split, row)
    assert _wsize(lib, 1, 256, 8, 160, [256] * 5) == 1 * 8 * 5 * 256 * (160 + 2) * 4
    # one frame of the 8^2 level: five splits of one tile; two frames of 16^2: four
    assert _wsize(lib, 1, 64, 8, 160, [64] * 5) == 1 * 8 * 5 * 64 * 162 * 4
    assert _wsize(lib, 2, 256, 8, 160, [256] * 5) == 2 * 8 * 4 * 256 * 162 * 4
    # 41 tiles, one workgroup, 40 rows (tiny partials): one tile per split
    assert _wsize(lib, 1, 40, 1, 160, [64, 1024, 1024, 512]) == 41 * 40 * 162 * 4
    # a single key tile has nothing to split; short contexts take their own kernel
    assert _wsize(lib, 1, 64, 8, 160, [64]) == 0
    assert _wsize(lib, 1, 64, 8, 160, [32]) == 0
    # invalid sizes report 0 (the call itself rejects them)
    assert _wsize(lib, 1, 256, 8, 48, [256] * 5) == 0
    assert _wsize(lib, 0, 256, 8, 160, [256] * 5) == 0
    assert lib.pl_refbank_attn_workspace_size(1, 256, 8, 160, None, 5) == 0


def test_attention_rejects_small_workspace(lib):
    # a one-frame 16^2 launch splits its keys and needs a workspace: too small
    # or NULL with bytes is rejected before any launch; misaligned is unsupported
    F, L, C, H = 1, 256, 1280, 8
    n = _wsize(lib, F, L, H, 160, [256] * 5)
    assert n > 0
    segs = _segs((ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000), 256, C, L * C),
                 *[(ctypes.c_void_p(0x3000000 + 0x100000 * i), ctypes.c_void_p(0x4000000 + 0x100000 * i), 256, C, 0)
                   for i in range(4)])
    def call(ws, nbytes):
        return B.pl_refbank_attn(ctypes.c_void_p(0x5000000), C, L * C, ctypes.c_void_p(0x6000000), C, L * C, F, L, H,
                                 160, segs, 5, 0.08, ws, nbytes, None)
    assert call(ctypes.c_void_p(0x9000000), n - 16) == B.PL_EINVAL and "too small" in B.last_error()
    assert call(None, n) == B.PL_EINVAL and "NULL" in B.last_error()
    assert call(ctypes.c_void_p(0x9000008), n) == B.PL_EUNSUPPORTED and "workspace" in B.last_error()


def _ddim(x=A, e=A, xp=A2, x0=A, W=4, n=256, t=(999, 666, 333, 0), step=333, ab=None, T=1000, fin=-1.0, emit=3):
    ts = (ctypes.c_int32 * max(1, len(t)))(*t)
    return B.pl_pyramid_ddim_step(x, e, xp, x0, W, n, ts, step, ab, T, fin, emit, None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(e=None), dict(xp=None), dict(W=0), dict(W=9), dict(n=0), dict(step=0),
    dict(t=(999, 666, 333, 1000)), dict(t=(999, 666, 333, -1)), dict(emit=4), dict(emit=-2),
    dict(x0=None), dict(T=999), dict(fin=1.5),
])
def test_ddim_rejects(lib, kw):
    assert _ddim(**kw) == B.PL_EINVAL
    assert B.last_error() != ""


def test_ddim_rejects_bad_schedule(lib):
    ab = (ctypes.c_double * 3)(0.9, 0.0, 0.5)
    assert _ddim(t=(2, 1, 0, 0), ab=ab, T=3) == B.PL_EINVAL
    assert "alphas_cumprod[1]" in B.last_error()


@pytest.mark.parametrize("kw", [dict(x=None), dict(W=0), dict(emit=4), dict(x0=None), dict(T=999)])
def test_ddim_roll_rejects(lib, kw):
    args = dict(x=A, e=A2, xp=A, x0=A2, W=4, n=65536, t=(999, 666, 333, 0), step=333, ab=None, T=1000,
                fin=-1.0, emit=3)
    args.update(kw)
    ts = (ctypes.c_int32 * 4)(*args["t"])
    st = B.pl_pyramid_ddim_step_roll(args["x"], args["e"], args["xp"], args["x0"], args["W"], args["n"], ts,
                                     args["step"], args["ab"], args["T"], args["fin"], args["emit"], 7, 11, None)
    assert st == B.PL_EINVAL
    assert B.last_error() != ""


def test_linear_rejects(lib):
    ok = dict(x=A, xld=320, w=A2, wld=320, b=None, y=ctypes.c_void_p(0x40000), yld=960, M=100, N=960, K=320)
    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return B.pl_linear(a["x"], a["xld"], a["w"], a["wld"], a["b"], a["y"], a["yld"], a["M"], a["N"], a["K"], None)
    assert call(x=None) == B.PL_EINVAL
    assert call(M=0) == B.PL_EINVAL
    assert call(N=100) == B.PL_EUNSUPPORTED
    assert call(K=40) == B.PL_EUNSUPPORTED
    assert call(xld=300) == B.PL_EINVAL
    assert call(yld=900) == B.PL_EINVAL
    assert call(x=MIS) == B.PL_EUNSUPPORTED
    assert call(y=ctypes.c_void_p(0x10000 + 2 * 320)) == B.PL_EINVAL  # y overlaps x
    assert "overlap" in B.last_error()


def test_noise_prefill_lerp_reject(lib):
    assert B.pl_window_noise(None, 16, 1, 2, None) == B.PL_EINVAL
    assert B.pl_window_noise(A, 0, 1, 2, None) == B.PL_EINVAL
    # prefill: null pointers, window count, the top window beyond the schedule, overlap
    assert B.pl_pile_prefill(None, A, 3, 64, 333, None, 1000, 5, None) == B.PL_EINVAL
    assert B.pl_pile_prefill(A2, A, 0, 64, 333, None, 1000, 5, None) == B.PL_EINVAL
    assert B.pl_pile_prefill(A2, A, 9, 64, 333, None, 1000, 5, None) == B.PL_EINVAL
    assert B.pl_pile_prefill(A2, A, 4, 64, 334, None, 1000, 5, None) == B.PL_EINVAL
    assert "t = 1002" in B.last_error()
    assert B.pl_pile_prefill(ctypes.c_void_p(0x10000 + 64 * 4), A, 3, 64, 333, None, 1000, 5, None) == B.PL_EINVAL
    assert "overlap" in B.last_error()
    assert B.pl_pile_prefill(A2, A, 3, 64, 333, None, 999, 5, None) == B.PL_EINVAL
    # lerp: null, sizes, overlap of out with an input
    assert B.pl_lerp_points(None, A2, 16, 12, A, None) == B.PL_EINVAL
    assert B.pl_lerp_points(A2, A2, 0, 12, A, None) == B.PL_EINVAL
    assert B.pl_lerp_points(A2, A2, 16, 0, A, None) == B.PL_EINVAL
    assert B.pl_lerp_points(A, A2, 16, 12, ctypes.c_void_p(0x10000 - 64), None) == B.PL_EINVAL
    assert "overlap" in B.last_error()


@pytest.mark.parametrize("kw", [
    dict(nq=0), dict(n=0), dict(n=5), dict(D=0), dict(D=65537), dict(q=None), dict(ex=None),
    dict(thr=float("nan")),
])
def test_motion_rejects(lib, kw):
    args = dict(q=A, nq=1, b=A2, n=4, D=512, thr=17.0, md=A, am=A, ex=A)
    args.update(kw)
    st = B.pl_motion_bank_min_l2(args["q"], args["nq"], args["b"], args["n"], args["D"], args["thr"], args["md"],
                                 args["am"], args["ex"], None)
    assert st == B.PL_EINVAL


def test_last_error_clears_after_success(lib):
    p = B.pl_pile()
    assert B.pl_pile_init(ctypes.byref(p), 1, 333, 0, 1) == B.PL_EINVAL
    assert B.last_error() != ""
    assert B.pl_pile_init(ctypes.byref(p), 4, 333, 999, 1) == B.PL_OK
    assert B.last_error() == ""


def test_pile_rejects(lib):
    p = B.pl_pile()
    assert B.pl_pile_init(ctypes.byref(p), 4, 333, 998, 1) == B.PL_EINVAL
    assert B.pl_pile_init(ctypes.byref(p), 9, 333, 8 * 333, 1) == B.PL_EINVAL
    assert B.pl_pile_init(ctypes.byref(p), 4, 0, 0, 1) == B.PL_EINVAL
    assert B.pl_pile_init(ctypes.byref(p), 4, 333, 999, 1) == B.PL_OK
    e = ctypes.c_int64()
    assert B.pl_pile_end_round(ctypes.byref(p), ctypes.byref(e)) == B.PL_EINVAL
    pile = B.Pile()
    pile.begin_round()
    with pytest.raises(B.PlError):
        pile.begin_round()


@pytest.mark.parametrize("prefill", [True, False])
def test_pile_matches_oracle_queue(lib, prefill, pages_constants):
    ts = pages_constants["timesteps"]
    W = pages_constants["windows"]
    pile = B.Pile(W, pages_constants["step_length"], prefill=prefill)
    ref = PyramidPile(ts, pages_constants["frames_per_window"], prefill=prefill)
    slot_of = {wid: s for s, wid in enumerate(pile.slot_ids()) if wid >= 0}
    for r in range(14):
        new_slot, t_slot, emit_slot = pile.begin_round()
        ids = pile.slot_ids()
        evaluated, emitted = ref.round()
        assert ids[new_slot] == evaluated[-1][0]
        slot_of[ids[new_slot]] = new_slot
        # every held window sits in its slot at the oracle's timestep
        for wid, t in evaluated:
            assert t_slot[slot_of[wid]] == t
        held = {wid for wid, _ in evaluated}
        assert {i for i in ids if i >= 0} == held
        if emitted is None:
            assert emit_slot == -1
        else:
            assert emit_slot == slot_of[emitted] and t_slot[emit_slot] == 0
        assert pile.end_round() == (-1 if emitted is None else emitted)


def test_sd_alphas_cumprod_table(lib):
    # the library's built-in schedule, read back through the ABI, is the oracle's
    import numpy as np
    from oracle import sd_scaled_linear_alphas_cumprod
    ab = (ctypes.c_double * 1000)()
    assert lib.pl_sd_alphas_cumprod(ab, 1000) == B.PL_OK
    assert np.max(np.abs(np.array(ab) - sd_scaled_linear_alphas_cumprod())) <= 1e-15
    assert lib.pl_sd_alphas_cumprod(ab, 999) == B.PL_EINVAL
    assert lib.pl_sd_alphas_cumprod(None, 1000) == B.PL_EINVAL


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), B.PL_EINVAL), (dict(x0=None), B.PL_EINVAL), (dict(pile=None), B.PL_EINVAL),
    (dict(ab=None), B.PL_EINVAL), (dict(W=1), B.PL_EINVAL), (dict(W=9), B.PL_EINVAL), (dict(n=0), B.PL_EINVAL),
    (dict(T=0), B.PL_EINVAL), (dict(fin=1.5), B.PL_EINVAL), (dict(fin=0.0), B.PL_EINVAL),
    (dict(n=258), B.PL_EUNSUPPORTED), (dict(x=MIS), B.PL_EUNSUPPORTED), (dict(x0=MIS), B.PL_EUNSUPPORTED),
    (dict(pile=ctypes.c_void_p(0x30004)), B.PL_EUNSUPPORTED),
])
def test_ddim_device_rejects(lib, kw, status):
    a = dict(x=A, e=A2, xp=A, x0=A2, W=4, n=256, pile=ctypes.c_void_p(0x30000), ab=ctypes.c_void_p(0x40000),
             T=1000, fin=-1.0)
    a.update(kw)
    st = B.pl_pyramid_ddim_step_device(a["x"], a["e"], a["xp"], a["x0"], a["W"], a["n"], a["pile"], a["ab"], a["T"],
                                       a["fin"], 7, None)
    assert st == status
    assert B.last_error() != ""


def test_noalloc_rejects_split_beyond_its_scratch(lib):
    # one frame of a 2048-row d = 160 level with a 4x bank: two splits of
    # 2048 rows x 8 heads need about 21 MB of partials, more than the 16 MiB
    # the library holds; rejected before any device call
    F, L, C, H = 1, 2048, 1280, 8
    assert _wsize(lib, F, L, H, 160, [L] * 5) > 16 << 20
    segs = _segs((ctypes.c_void_p(0x10000000), ctypes.c_void_p(0x20000000), L, C, L * C),
                 *[(ctypes.c_void_p(0x30000000 + 0x1000000 * i), ctypes.c_void_p(0x40000000 + 0x1000000 * i), L, C, 0)
                   for i in range(4)])
    st = B.pl_refbank_attn_noalloc(ctypes.c_void_p(0x50000000), C, L * C, ctypes.c_void_p(0x60000000), C, L * C, F,
                                   L, H, 160, segs, 5, 0.08, None)
    assert st == B.PL_EINVAL and "scratch" in B.last_error()
    # argument checks are those of pl_refbank_attn
    assert B.pl_refbank_attn_noalloc(None, C, L * C, ctypes.c_void_p(0x60000000), C, L * C, F, L, H, 160, segs, 5,
                                     0.08, None) == B.PL_EINVAL


def test_chunked_rejects(lib):
    # (fake addresses, never dereferenced; every case fails validation)
    F, L, C, H = 2, 100, 64, 2
    q, o = ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000)
    ok = _segs((ctypes.c_void_p(0x3000000), ctypes.c_void_p(0x4000000), L, C, L * C),
               (ctypes.c_void_p(0x5000000), ctypes.c_void_p(0x6000000), 7, C, 0))
    def call(segs=ok, nseg=2, causal=0, cl=32, hist=-1, Lq=L, q_=q, o_=o):
        return B.pl_refbank_attn_chunked(q_, C, Lq * C, o_, C, Lq * C, F, Lq, H, 32, segs, nseg, causal, cl, hist,
                                         0.17, None)
    assert call(causal=2) == B.PL_EINVAL and "causal_seg" in B.last_error()
    assert call(causal=-1) == B.PL_EINVAL
    assert call(cl=0) == B.PL_EINVAL
    assert call(Lq=99) == B.PL_EINVAL and "Lq" in B.last_error()  # the causal segment holds 100 rows
    assert call(q_=None) == B.PL_EINVAL
    assert call(o_=ctypes.c_void_p(0x3000000)) == B.PL_EINVAL and "overlaps" in B.last_error()
    assert call(segs=None) == B.PL_EINVAL
    assert call(nseg=9) == B.PL_EINVAL
