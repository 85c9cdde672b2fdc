"""Oracle of the atomic-expert layer (OmniMoE page, technical summary 2.1 and
2.2). Test infrastructure only: imported by the tests, never by the library.
Plain fp64 NumPy, written from the definitions:

- atomic expert i (2.1): E_i(x) = sigma(x . w_in_i) w_out_i, with w_in_i and
  w_out_i the i-th rows of the global matrices W and V; sigma is read as SiLU,
  z / (1 + e^-z) (the page leaves the activation unnamed);
- Cartesian product router (2.2): the N = n_rows x n_cols experts form a grid,
  expert i = a * n_cols + b; row logits l_r = x . R_r^T and column logits
  l_c = x . R_c^T combine into the score s_i = l_r[a] + l_c[b];
- the k best scores win (ties to the lower index), weighted by the softmax
  over the k selected scores; y = sum_j w_j E_{i_j}(x).
"""
import numpy as np


def bf16_bits_to_f32(b) -> np.ndarray:
    """bfloat16 bit patterns (uint16) widened exactly to float32: the pattern
    is the upper half of the float32 pattern."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def scores(lr: np.ndarray, lc: np.ndarray, dtype=np.float64) -> np.ndarray:
    """[T][n_rows * n_cols] scores l_r[a] + l_c[b] in `dtype` (float32 sums
    reproduce the GPU's fp32 scores exactly)."""
    lr = np.asarray(lr, dtype)
    lc = np.asarray(lc, dtype)
    return (lr[:, :, None] + lc[:, None, :]).reshape(lr.shape[0], -1)


def topk(s: np.ndarray, k: int):
    """Selection by the definition: order every expert by (-score, index) and
    take the first k. Returns idx [T][k], softmax weights [T][k] in fp64 and the
    k-th minus (k+1)-th score (+inf when k = N)."""
    order = np.argsort(-s, axis=1, kind="stable")   # stable: equal scores keep ascending index
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(s, idx, axis=1).astype(np.float64)
    p = np.exp(sel - sel[:, :1])
    w = p / p.sum(axis=1, keepdims=True)
    if k < s.shape[1]:
        nxt = np.take_along_axis(s, order[:, k:k + 1], axis=1)[:, 0].astype(np.float64)
        margin = sel[:, -1] - nxt
    else:
        margin = np.full(s.shape[0], np.inf)
    return idx, w, margin


def silu(z):
    return z / (1.0 + np.exp(-z))


def layer(x_bits, w_in_bits, w_out_bits, rr_bits, rc_bits, k: int, given=None):
    """fp64 forward: dict(y, lr, lc, idx, w, margin). `given` [T][k] replaces the
    selection (its weights still come from the fp64 scores)."""
    X = bf16_bits_to_f32(x_bits).astype(np.float64)
    W = bf16_bits_to_f32(w_in_bits).astype(np.float64)
    V = bf16_bits_to_f32(w_out_bits).astype(np.float64)
    lr = X @ bf16_bits_to_f32(rr_bits).astype(np.float64).T
    lc = X @ bf16_bits_to_f32(rc_bits).astype(np.float64).T
    s = scores(lr, lc)
    idx, w, margin = topk(s, k)
    if given is not None:
        idx = np.asarray(given, np.int32)
        sel = np.take_along_axis(s, idx, axis=1)
        p = np.exp(sel - sel.max(axis=1, keepdims=True))
        w = p / p.sum(axis=1, keepdims=True)
    y = np.zeros_like(X)
    for j in range(k):
        e = idx[:, j]
        h = silu(np.einsum("td,td->t", X, W[e]))
        y += (w[:, j] * h)[:, None] * V[e]
    return dict(y=y, lr=lr, lc=lc, idx=idx, w=w, margin=margin)
