"""Base projection and gated LoRA of R-ISD (oracle side).

Test infrastructure, plain numpy in float64; it shares no code with the HIP
path. The pages fix that the lossless variant adds a LoRA adapter (rank 128
in the released model) only at MASK positions, so that the outputs at clean
positions stay bit-for-bit those of the base AR model (I-DLM,
fr.news.hada.io, "Speedup Factor Explorer" and "Documentation et ressources >
Lossless R-ISD"; overhead about 1.12x).

Readings where the pages are silent: the adapter is the usual low-rank
update y += s * (x A^T) B^T with A [r, K], B [Nout, r] and scale s; rank and
scale are parameters.
"""

import numpy as np


def linear(x, W):
    """y = x W^T, float64."""
    return np.asarray(x, np.float64) @ np.asarray(W, np.float64).T


def gated_lora(x, W, A, B, is_mask, scale):
    """y = x W^T on every row, plus scale * (x A^T) B^T on MASK rows only."""
    x = np.asarray(x, np.float64)
    y = linear(x, W)
    m = np.asarray(is_mask, bool)
    if m.any():
        t = x[m] @ np.asarray(A, np.float64).T
        y[m] = y[m] + scale * (t @ np.asarray(B, np.float64).T)
    return y
