"""Key-segment lists of the bounded-context schemes (host logic, CPU)."""

import numpy as np
import pytest

from streaming_diffusion_portrait_amd.context import (sink_window_ids, pr_sink_ids, dynamic_sink_candidates,
                                                       context_segments)


def test_sink_window_steady_state_is_three_sinks_and_two_recent():
    assert sink_window_ids(10) == [0, 1, 2, 8, 9]
    assert sink_window_ids(1000) == [0, 1, 2, 998, 999]
    # context size is bounded: 5 chunks for every chunk after the first five
    assert all(len(sink_window_ids(c)) == 5 for c in range(5, 200))


def test_sink_window_start_of_stream_never_repeats_or_looks_ahead():
    assert sink_window_ids(0) == []
    assert sink_window_ids(1) == [0]
    assert sink_window_ids(3) == [0, 1, 2]
    assert sink_window_ids(4) == [0, 1, 2, 3]
    for c in range(0, 50):
        ids = sink_window_ids(c)
        assert len(ids) == len(set(ids))
        assert all(0 <= i < c for i in ids)  # chunk-causal: only earlier chunks


def test_pr_sink_static_dynamic_and_buffer():
    assert pr_sink_ids(10, dynamic=4) == [0, 4, 7, 8, 9]
    assert pr_sink_ids(10) == [0, 7, 8, 9]
    assert pr_sink_ids(10, dynamic=8) == [0, 7, 8, 9]   # already in the buffer: not repeated
    assert pr_sink_ids(2, dynamic=0) == [0, 1]
    assert pr_sink_ids(0) == []
    with pytest.raises(ValueError):
        pr_sink_ids(5, dynamic=5)
    assert dynamic_sink_candidates(10) == [1, 2, 3, 4, 5, 6]
    assert dynamic_sink_candidates(3) == []


def test_context_segments_order():
    cur, ref = ("kc", "vc"), ("kr", "vr")
    cache = {i: (f"k{i}", f"v{i}") for i in range(6)}
    assert context_segments(cur, cache, [0, 4], ref) == [cur, cache[0], cache[4], ref]
    assert context_segments(cur, cache, [], None) == [cur]
