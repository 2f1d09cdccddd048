"""Oracle for the segment-masked short causal convolution.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows RFC-0025, Design section 3 ("ShortConvolution segment boundary
mask"): a causal depthwise convolution of width Kc in which tap k multiplies
the input k positions back, and a tap is zeroed when its source position
belongs to another segment than the output position (the left padding counts
as id 0). No bias and no activation. Tap order: ``w[f, k]`` is the page's
``kernel[k]`` for channel f, so ``w[:, 0]`` weights the current token.
"""

import numpy as np


def short_conv_segmask(x, w, segment_ids=None):
    """y[b, t, f] = sum_k w[f, k] * x[b, t - k, f] * [t - k >= 0] * [seg[b, t - k] == seg[b, t]].

    x: [B, T, F]; w: [F, Kc]; segment_ids: [B, T] or None (no mask).
    Returns float64 [B, T, F].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, F = x.shape
    Fw, Kc = w.shape
    if Fw != F:
        raise ValueError("w must be [F, Kc]")
    seg = None if segment_ids is None else np.asarray(segment_ids).astype(np.int64)
    y = np.zeros((B, T, F), dtype=np.float64)
    for b in range(B):
        for t in range(T):
            acc = np.zeros(F, dtype=np.float64)
            for k in range(Kc):
                src = t - k
                if src < 0:
                    continue
                if seg is not None and seg[b, src] != seg[b, t]:
                    continue
                acc += w[:, k] * x[b, src, :]
            y[b, t, :] = acc
    return y
