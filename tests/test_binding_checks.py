"""CPU tests of the Python binding's own argument checks: shapes the C ABI
cannot see (a segment's frame count and width, the extent of a projection's
output) are rejected before anything reaches the library."""

import pytest

torch = pytest.importorskip("torch")

from streaming_diffusion_portrait_amd import binding as B  # noqa: E402


def _kv(*shape):
    t = torch.zeros(*shape, dtype=torch.float16)
    return t, torch.zeros_like(t)


def test_segment_frame_count_must_match_q():
    with pytest.raises(ValueError, match="frames"):
        B.make_segments([_kv(4, 8, 64)], frames=16, channels=64)


def test_segment_width_must_match_q():
    with pytest.raises(ValueError, match="columns"):
        B.make_segments([_kv(16, 8, 32)], frames=16, channels=64)
    with pytest.raises(ValueError, match="columns"):
        B.make_segments([_kv(8, 128)], frames=16, channels=64)


def test_segment_k_v_must_agree():
    k = torch.zeros(16, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="share shape"):
        B.make_segments([(k, torch.zeros(16, 9, 64, dtype=torch.float16))], frames=16, channels=64)


def test_shape_checks_pass_before_the_device_check():
    # a well-formed table of host tensors gets as far as the device check:
    # a one-frame [1, L, C] segment is accepted as shared, [F, L, C] as per-frame
    for segs in ([_kv(1, 8, 64)], [_kv(16, 8, 64)], [_kv(8, 64)]):
        with pytest.raises(TypeError, match="device tensor"):
            B.make_segments(segs, frames=16, channels=64)


def test_linear_out_shape_checked():
    x = torch.zeros(100, 64, dtype=torch.float16)
    w = torch.zeros(128, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="out must have shape"):
        B.linear(x, w, out=torch.zeros(50, 128, dtype=torch.float16))  # too few rows
    with pytest.raises(ValueError, match="out must have shape"):
        B.linear(x, w, out=torch.zeros(100, 64, dtype=torch.float16))  # too few columns
    x3 = torch.zeros(2, 50, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="out must have shape"):
        B.linear(x3, w, out=torch.zeros(100, 128, dtype=torch.float16))  # rank differs


def test_linear_rejects_outputs_that_are_not_one_matrix():
    # [2, 50, 128] inside a taller [2, 60, 128] buffer: its rows are not evenly
    # spaced, so it cannot be written as one [100, 128] matrix -- a reshape
    # would return a copy and the results would never reach the caller's buffer
    x3 = torch.zeros(2, 50, 64, dtype=torch.float16)
    w = torch.zeros(128, 64, dtype=torch.float16)
    buf = torch.zeros(2, 60, 128, dtype=torch.float16)
    with pytest.raises(ValueError, match="one row stride"):
        B.linear(x3, w, out=buf[:, :50, :])
    xbuf = torch.zeros(2, 60, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="one row stride"):
        B.linear(xbuf[:, :50, :], w)


def test_linear_accepts_well_formed_views_up_to_the_device_check():
    x3 = torch.zeros(2, 50, 64, dtype=torch.float16)
    w = torch.zeros(128, 64, dtype=torch.float16)
    with pytest.raises(TypeError, match="device tensor"):
        B.linear(x3, w, out=torch.zeros(2, 50, 128, dtype=torch.float16))
