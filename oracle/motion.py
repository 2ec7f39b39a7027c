"""Oracle: the motion-bank minimum-L2 drift check, in fp64.

Test infrastructure only (see the package docstring).

PersonaLive write-up, section "抗身份漂移的补丁" (anti identity-drift patch):
the expression embedding of the current frame is compared with the motion
bank; when the smallest L2 distance exceeds 17 the current clean frame is run
through the Reference UNet again and its layer features join the bank, at
most three times per stream.  Section "三条条件通路" gives the embedding: the
MotEncoder's 512-dimensional output.

Readings (listed in the design notes): "L2 distance" is the Euclidean norm
(not squared); "exceeds" is strict ``>``; argmin takes the lowest index on
ties.  The append policy (cap of three) belongs to the caller.
"""

import numpy as np


def motion_bank_min_l2(query, bank, threshold=17.0):
    """Minimum Euclidean distance of each query to the bank entries.

    ``query`` [nq, D] (or [D]), ``bank`` [n, D].  Returns
    ``(min_dist [nq] float64, argmin [nq] int64, exceeds [nq] bool)`` with
    ``exceeds = min_dist > threshold``.
    """
    q = np.atleast_2d(np.asarray(query, dtype=np.float64))
    b = np.atleast_2d(np.asarray(bank, dtype=np.float64))
    if q.shape[1] != b.shape[1] or b.shape[0] < 1:
        raise ValueError("query and bank must share D and the bank must be non-empty")
    diff = q[:, None, :] - b[None, :, :]
    dist = np.sqrt(np.sum(diff * diff, axis=2))
    arg = np.argmin(dist, axis=1)  # numpy returns the first (lowest) index on ties
    mind = dist[np.arange(q.shape[0]), arg]
    return mind, arg.astype(np.int64), mind > float(threshold)
