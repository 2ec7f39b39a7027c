"""Oracle: reference-bank spatial self-attention, plain definition in fp64.

Test infrastructure only (see the package docstring).

What is computed (PersonaLive write-up, section "三条条件通路" / three
conditioning paths): the Reference UNet stores each layer's features in a
bank; the denoising UNet concatenates that layer's bank features with its own
keys/values and runs ordinary spatial self-attention over the result.  The
bank is encoded once and reused for the whole stream, so it is shared by all
frames of the 16-frame batch; anchors appended by the drift check (section
"抗身份漂移的补丁") add further bank entries of the same shape.

For frame f and head h, with d = C / heads and scale = 1/sqrt(d) unless given::

    K_cat = concat_s K_s[f or shared][:, h*d:(h+1)*d]      (over segments s)
    V_cat = concat_s V_s[f or shared][:, h*d:(h+1)*d]
    S     = Q[f][:, h*d:(h+1)*d] @ K_cat.T * scale
    P     = softmax(S, axis=keys)                            (max-subtracted)
    O[f][:, h*d:(h+1)*d] = P @ V_cat

No mask, dropout or bias.  A flash / online evaluation reaches exactly this
result up to rounding, so the oracle is the definition written out with a
library matmul as the only primitive.
"""

import numpy as np


def _segment_frame(arr, shared, f):
    """Rows of one segment as seen by frame ``f``.

    A per-frame segment is ``[F, Ls, C]`` and frame f reads slice f; a shared
    (bank) segment is ``[Ls, C]`` and every frame reads the same rows.
    """
    a = np.asarray(arr)
    return a if shared else a[f]


def concat_segments(segments, f):
    """Concatenate the key and value rows of all segments for frame ``f``.

    ``segments`` is a sequence of ``(k, v, shared)``.  Returns fp64
    ``(K_cat, V_cat)`` with shape ``[sum Ls, C]``.
    """
    ks = [np.asarray(_segment_frame(k, shared, f), dtype=np.float64) for k, _, shared in segments]
    vs = [np.asarray(_segment_frame(v, shared, f), dtype=np.float64) for _, v, shared in segments]
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def attend_rows(q_rows, k_cat, v_cat, scale):
    """softmax(q_rows @ k_cat.T * scale) @ v_cat for one head, in fp64.

    ``q_rows`` [n, d], ``k_cat`` [Lk, d], ``v_cat`` [Lk, d].  The row maximum
    is subtracted before the exponential (standard softmax definition).
    """
    q = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k_cat, dtype=np.float64)
    v = np.asarray(v_cat, dtype=np.float64)
    s = (q @ k.T) * float(scale)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def refbank_attention(q, segments, heads, scale=None, frames=None, head_list=None, rows=None):
    """Reference-bank spatial self-attention over a segment list, in fp64.

    Parameters
    ----------
    q : array [F, L, C]
        Queries, token-major; head h occupies columns ``[h*d, (h+1)*d)``.
    segments : sequence of (k, v, shared)
        Key/value sources in key order.  ``shared=False``: ``[F, Ls, C]``,
        one slice per frame (the frame's own tokens).  ``shared=True``:
        ``[Ls, C]``, the same rows for every frame (reference / anchors).
    heads : int
        Number of heads H; d = C / H.
    scale : float, optional
        Logit scale, default 1/sqrt(d).
    frames, head_list, rows : optional
        Restrict the computation to these frames / heads / query rows (the
        definition is row-wise, so a restriction computes exactly the same
        values for the rows it keeps).  Returns a dict
        ``{(f, h): [len(rows), d]}`` when any restriction is given.

    Returns
    -------
    ndarray [F, L, C] float64, or the dict described above.
    """
    q = np.asarray(q)
    F, L, C = q.shape
    if C % heads:
        raise ValueError("C must be divisible by heads")
    d = C // heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    restricted = frames is not None or head_list is not None or rows is not None
    fr = range(F) if frames is None else frames
    hs = range(heads) if head_list is None else head_list
    rr = np.arange(L) if rows is None else np.asarray(rows)
    if restricted:
        out = {}
    else:
        out = np.empty((F, L, C), dtype=np.float64)
    for f in fr:
        k_cat, v_cat = concat_segments(segments, f)
        qf = np.asarray(q[f], dtype=np.float64)
        for h in hs:
            cols = slice(h * d, (h + 1) * d)
            o = attend_rows(qf[rr][:, cols], k_cat[:, cols], v_cat[:, cols], scale)
            if restricted:
                out[(f, h)] = o
            else:
                out[f][:, cols] = o
    return out


def chunk_causal_attention(q, self_kv, shared, heads, chunk_len, max_history=-1, scale=None):
    """Block-causal attention over one token sequence per frame, in fp64.

    Deep-compression-VAE write-up (papernotes) and LPM write-up, section 6.3
    分块因果注意力: the sequence is cut into non-overlapping chunks of
    ``chunk_len`` tokens; a token attends to every token of its own chunk and
    of earlier chunks (at most ``max_history`` of them; negative = all), never
    to a later chunk, and to the persistent reference tokens.

    ``q``: [F, L, C]; ``self_kv``: (k, v) [F, L, C], row j of frame f in chunk
    j // chunk_len; ``shared``: list of (k, v) [Ls, C] visible to every row.
    Returns [F, L, C] fp64.  Plain definition: the visible keys of each row are
    gathered and the row is attended with :func:`attend_rows`.
    """
    q = np.asarray(q)
    F, L, C = q.shape
    d = C // heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    ks, vs = (np.asarray(a, dtype=np.float64) for a in self_kv)
    sk = [np.asarray(k, dtype=np.float64) for k, _ in shared]
    sv = [np.asarray(v, dtype=np.float64) for _, v in shared]
    out = np.empty((F, L, C), dtype=np.float64)
    for f in range(F):
        for r in range(L):
            c = r // chunk_len
            lo = 0 if max_history < 0 else max(0, c - max_history)
            rows = np.arange(lo * chunk_len, min(L, (c + 1) * chunk_len))
            kcat = np.concatenate([ks[f][rows]] + sk, axis=0)
            vcat = np.concatenate([vs[f][rows]] + sv, axis=0)
            qf = np.asarray(q[f][r:r + 1], dtype=np.float64)
            for h in range(heads):
                cols = slice(h * d, (h + 1) * d)
                out[f, r, cols] = attend_rows(qf[:, cols], kcat[:, cols], vcat[:, cols], scale)[0]
    return out
