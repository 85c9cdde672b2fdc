"""Whole-batch evaluation of a layer's definition with library matmuls, for
pinning how the output's rounding interacts with the max-abs bar on complete
outputs (test infrastructure).

The layer (Q-MoE page, section 3: gating network, quantized experts, sparse
execution; FineRMoE architecture paragraph: SwiGLU experts mixed by the
router's softmax probabilities, shared experts added with weight 1) is
evaluated here per expert over all of its tokens with fp64 matrix products on
the oracle's dequantized weights. It is tied to the oracle itself by a test
that compares both on sampled tokens; its only purpose is to emulate the
roundings the GPU path is allowed (bf16 H before the down projection, the
expert outputs' 16-bit block codes, bf16 y) on complete full-size outputs,
where the per-token oracle would take minutes.
"""
from __future__ import annotations

import numpy as np

from quantized_mixture_experts_qmoe_amd.inputs import bf16_bits_to_f32


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even) via float32, as float64.
    The float64 -> float32 step rounds first; it is exact for every value this
    is applied to at the precision that matters here (2^-24 relative)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.view(np.float32).astype(np.float64)


def o_code_round(v: np.ndarray) -> np.ndarray:
    """The expert outputs' storage between the down projection and the sum:
    per row and 16 consecutive columns, with e the exponent of the block's
    largest |v| (|v|max in [2^(e-1), 2^e)), the code q = round(32767 * v / 2^e)
    and the value read back q * (2^e / 32767), in float32 as the path computes
    it. Rows of v are the outputs of one (token, expert) pair; the column count
    is a multiple of 16."""
    f = np.ascontiguousarray(v, dtype=np.float32)
    b = f.reshape(f.shape[0], -1, 16)
    amax = np.abs(b).max(axis=2, keepdims=True)
    e = np.clip(np.frexp(amax)[1], -126, 127).astype(np.int32)
    scaled = (b * np.ldexp(np.float32(1.0), -e).astype(np.float32)).astype(np.float32)
    q = np.rint(np.clip(scaled, -1.0, 1.0) * np.float32(32767.0)).astype(np.float32)
    back = q * np.ldexp(np.float32(1.0 / 32767.0), e).astype(np.float32)
    return back.reshape(f.shape).astype(np.float64)


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |v| (8 significant bits)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def routing(inp):
    """fp64 logits, top-k by (descending logit, ascending index) and the
    softmax over the selected k (renormalised) for every token."""
    cfg = inp.cfg
    X = bf16_bits_to_f32(inp.x).astype(np.float64)
    Wr = (inp.w_router if cfg.router_fp32 else bf16_bits_to_f32(inp.w_router)).astype(np.float64)
    L = X @ Wr.T + (0.0 if inp.bias is None else inp.bias.astype(np.float64))
    idx = np.argsort(-L, axis=1, kind="stable")[:, :cfg.k]
    sel = np.take_along_axis(L, idx, axis=1)
    p = np.exp(sel - sel[:, :1])
    assert cfg.renormalize
    return X, L, idx, p / p.sum(1, keepdims=True)


def exact_and_path(O, layer, inp):
    """(y_exact, y_path): the layer in fp64 on every token, and the same with
    the path's storage roundings applied (H rounded to bf16 before the down
    projection; each expert output in its 16-bit block code; the summed output
    rounded once to bf16)."""
    cfg = inp.cfg
    X, _, idx, w = routing(inp)
    T = X.shape[0]
    y = np.zeros((T, cfg.d))
    yp = np.zeros((T, cfg.d))
    for e in range(cfg.E + cfg.S):
        if e < cfg.E:
            tt, jj = np.nonzero(idx == e)
            if tt.size == 0:
                continue
            mix = w[tt, jj][:, None]
        else:
            tt = np.arange(T)
            mix = 1.0
        fe = cfg.expert_format(e)
        Wg = O.dequantize(fe, *layer.codes(e, 0), group=cfg.group)
        Wu = O.dequantize(fe, *layer.codes(e, 1), group=cfg.group)
        Xe = X[tt]
        g = Xe @ Wg.T
        del Wg
        u = Xe @ Wu.T
        del Wu
        h = g / (1.0 + np.exp(-g)) * u
        del g, u
        Wd = O.dequantize(fe, *layer.codes(e, 2), group=cfg.group)
        # a token picks an expert at most once: tt has no repeats
        y[tt] += mix * (h @ Wd.T)
        yp[tt] += o_code_round(mix * (bf16_round(h) @ Wd.T))
        del Wd, h
    return y, bf16_round(yp)
