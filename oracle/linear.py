"""Oracle: the projections either side of the attention (to_q / to_k / to_v,
the bank's K/V projection and to_out), in fp64.

Test infrastructure only (see the package docstring).

PersonaLive write-up, section "三条条件通路": the Reference UNet stores each
layer's ``norm_hidden_states`` in the bank, and the denoiser joins those
features to its own keys and values; the keys and values are therefore the
layer's linear projections of those hidden states (projecting the bank once,
when it is written, gives the same keys as projecting the joined sequence --
a projection acts on each token separately).  The projections are plain
linear layers, ``y = x W^T (+ b)``, with W stored as [out features, in
features].

The oracle is that definition: a matrix product of the fp16-rounded inputs
in fp64 (NumPy's matmul serves as the step), plus the bias.
"""

import numpy as np


def linear(x, w, bias=None):
    """y[m, n] = sum_k x[m, k] * w[n, k] (+ bias[n]), fp64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y
