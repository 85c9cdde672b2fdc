"""Routing-shift metrics: how a change of router moves each token's top-k
selection, measured against a reference router on the same tokens.

The Q-MoE page (section 4) lists quantized routing among the quantization
options; the IT Donga article (DREAM-MoE section) explains why it is delicate:
when the k-th and (k+1)-th logits of a token are close, a small perturbation
of the logits, such as the one a quantized router weight brings, swaps an
expert in or out of the selection. These metrics count such swaps and place
them against the reference router's margins. Host-side arithmetic on routing
results the library returns (no part of the layer's computation)."""
from typing import Dict, Optional

import numpy as np

# reference-margin bins of the histograms: [0, 1e-3), [1e-3, 1e-2), ...
MARGIN_EDGES = (0.0, 1e-3, 1e-2, 1e-1, 1.0, np.inf)


def topk_margin(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token: the k-th largest logit minus the (k+1)-th (+inf when k = E)."""
    lg = np.asarray(logits, np.float64)
    if k >= lg.shape[1]:
        return np.full(lg.shape[0], np.inf)
    part = -np.sort(-lg, axis=1)
    return part[:, k - 1] - part[:, k]


def routing_shift(idx_ref: np.ndarray, idx_new: np.ndarray, logits_ref: np.ndarray,
                  margin: Optional[np.ndarray] = None) -> Dict[str, object]:
    """Compare two top-k selections [T][k] of the same tokens.

    Returns the number of tokens whose selected set differs (set_flips) and its
    rate, the number of selected experts replaced over all tokens
    (experts_swapped), the tokens with the same set in another slot order
    (order_changes), histograms over MARGIN_EDGES of the reference router's
    k-th/(k+1)-th margin for all tokens and for the flipped ones, and the
    largest reference margin among flipped tokens."""
    idx_ref = np.asarray(idx_ref)
    idx_new = np.asarray(idx_new)
    assert idx_ref.shape == idx_new.shape and idx_ref.ndim == 2
    T, k = idx_ref.shape
    m = topk_margin(logits_ref, k) if margin is None else np.asarray(margin, np.float64)
    flipped = np.zeros(T, bool)
    swapped = 0
    order = 0
    for t in range(T):
        a, b = set(idx_ref[t].tolist()), set(idx_new[t].tolist())
        if a != b:
            flipped[t] = True
            swapped += len(a - b)
        elif not np.array_equal(idx_ref[t], idx_new[t]):
            order += 1
    edges = np.asarray(MARGIN_EDGES)
    hist_all = np.histogram(np.minimum(m, 1e300), bins=edges)[0]
    hist_flip = np.histogram(np.minimum(m[flipped], 1e300), bins=edges)[0]
    return dict(tokens=T, set_flips=int(flipped.sum()), flip_rate=float(flipped.mean()) if T else 0.0,
                experts_swapped=int(swapped), order_changes=int(order),
                margin_edges=list(MARGIN_EDGES), margin_hist_all=hist_all.tolist(),
                margin_hist_flipped=hist_flip.tolist(),
                max_flipped_margin=float(m[flipped].max()) if flipped.any() else 0.0,
                flipped_tokens=np.nonzero(flipped)[0])
