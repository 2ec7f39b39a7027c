"""Which cached chunks a streaming chunk attends to: the key-segment lists of
chunk-causal attention with sink, sliding-window and pose-retrieval caches.

Host logic only (it picks chunk ids; the attention itself is one
``pl_refbank_attn`` call over the chosen segments, nothing is copied).

The pages describe three bounded-context schemes that differ only in which
earlier chunks are kept as keys:

* chunk-causal attention (LPM write-up, section 6.3 分块因果注意力): a
  chunk's tokens see the current chunk, a limited number of earlier chunks
  and the persistent reference tokens, never a later chunk;
* sink + sliding window (same write-up, section 7.3 滑动窗口注意力): 3 fixed
  sink chunks, 2 sliding-window chunks and the reference tokens, so the
  context per chunk stays the same size however long the session runs;
* PR-Sink (LiveAnimate summary): a static sink (the first generated chunk),
  one dynamic sink retrieved by pose match among earlier chunks, and a
  sliding buffer of three chunks.

Readings: "sink chunks" are the first chunks of the stream; the sliding window
holds the chunks right before the current one, without repeating a sink; the
dynamic sink is the earlier chunk (outside the window and the static sink)
whose pose embedding is nearest in L2 to the current chunk's, lowest id on
ties -- the same minimum-L2 rule as the motion-bank check, so it can be taken
from ``pl_motion_bank_min_l2``'s argmin.
"""


def sink_window_ids(current, n_sink=3, n_window=2):
    """Earlier chunk ids a chunk attends to, oldest first: sinks, then the window."""
    if current < 0 or n_sink < 0 or n_window < 0:
        raise ValueError("chunk ids and counts must be non-negative")
    sinks = list(range(min(n_sink, current)))
    window = [c for c in range(max(0, current - n_window), current) if c not in sinks]
    return sinks + window


def pr_sink_ids(current, dynamic=None, n_window=3):
    """Earlier chunk ids for PR-Sink: the static sink (chunk 0), the dynamic sink
    (``dynamic``, if given and not already kept) and the sliding buffer."""
    if current < 0 or n_window < 0:
        raise ValueError("chunk ids and counts must be non-negative")
    keep = [0] if current > 0 else []
    window = [c for c in range(max(0, current - n_window), current) if c not in keep]
    if dynamic is not None:
        if not 0 <= dynamic < current:
            raise ValueError("the dynamic sink must be an earlier chunk")
        if dynamic not in keep and dynamic not in window:
            keep.append(dynamic)
    return keep + window


def dynamic_sink_candidates(current, n_window=3):
    """Chunks the pose retrieval may choose from: earlier, not the static sink,
    not in the sliding buffer."""
    return [c for c in range(1, max(1, current - n_window))]


def context_segments(current_kv, cached_kv, ids, reference_kv=None):
    """Segment list for one chunk: its own K/V first, the chosen cached chunks,
    then the reference tokens (the order does not change the result).

    ``current_kv``: (k, v) of the current chunk ([1, L, C] per-frame tensors);
    ``cached_kv``: mapping chunk id -> (k, v) ([L, C], shared);
    ``reference_kv``: (k, v) of the persistent reference tokens, or None.
    """
    segs = [current_kv] + [cached_kv[c] for c in ids]
    if reference_kv is not None:
        segs.append(reference_kv)
    return segs
