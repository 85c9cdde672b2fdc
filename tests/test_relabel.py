"""Expert relabelling invariance.

Which integer names an expert is arbitrary: the layer (Q-MoE page, section 3:
the gating network's top-k selection over expert scores, the quantized experts
and the sparse execution that mixes their outputs) depends on the experts only
through their weights and router rows. Renaming the routed experts by a
permutation pi (router row i and expert i of the new layer are router row
pi[i] and expert pi[i] of the old one) must leave every output unchanged, and
turn each selected index e into pi^-1[e] (as long as no two of a token's
scores tie exactly, which the tests check: equal scores are ordered by index).
The oracle evaluates each (token, expert) pair with the same arithmetic
wherever the expert sits in the list, but adds a token's expert outputs in
expert order, so its outputs agree to fp64 rounding; the HIP path adds them in
selection order, so its outputs are equal bit for bit.
"""
import dataclasses

import numpy as np
import pytest

from quantized_mixture_experts_qmoe_amd.inputs import CONFIGS, LayerConfig, make_inputs


def relabel(inp, pi):
    """The same layer with routed expert i renamed pi^-1[i] (new expert i is old expert pi[i])."""
    cfg = inp.cfg
    E = cfg.E
    fmts = cfg.expert_formats
    if fmts is not None:
        fmts = tuple(fmts[p] for p in pi) + tuple(fmts[E:])
    new_cfg = cfg.replace(name=cfg.name + "_relabelled", expert_formats=fmts)
    order = list(pi) + list(range(E, E + cfg.S))
    return dataclasses.replace(
        inp, cfg=new_cfg, w_router=np.ascontiguousarray(inp.w_router[pi]),
        bias=None if inp.bias is None else np.ascontiguousarray(inp.bias[pi]),
        w_gate=[inp.w_gate[i] for i in order], w_up=[inp.w_up[i] for i in order],
        w_down=[inp.w_down[i] for i in order])


def small_cfg(fmt, **kw):
    base = dict(name=f"relabel_{fmt}", T=200, d=512, E=16, k=4, F=256, wformat=fmt,
                router_fp32=(fmt == "int8_sym_ch"))
    base.update(kw)
    return LayerConfig(**base)


ORACLE_CASES = [
    small_cfg("int4_asym_g128", bias=True),
    small_cfg("int3_sym_g128", S=1, Fs=256),
    small_cfg("fp8e4m3_ch", router_quant="int8"),
    small_cfg("int4_sym_g128", expert_formats=tuple(("int8_sym_ch", "int4_sym_g128", "fp8e4m3_ch",
                                                     "int4_asym_g128")[e % 4] for e in range(16))),
]


@pytest.mark.parametrize("cfg", ORACLE_CASES, ids=lambda c: c.name + "_" + c.wformat)
def test_oracle_expert_relabelling_invariance(oracle_mod, cfg):
    O = oracle_mod
    inp = make_inputs(cfg, seed=11)
    pi = np.random.default_rng(5).permutation(cfg.E)
    a = O.OracleLayer(inp)
    b = O.OracleLayer(relabel(inp, pi))
    ra, rb = a.forward(inp.x), b.forward(inp.x)
    a.close()
    b.close()
    # no exact tie among a token's scores (the order among equal scores
    # follows the index, which the renaming changes)
    s = np.sort(ra["logits"], axis=1)
    assert (np.diff(s, axis=1) != 0).all()
    assert np.array_equal(rb["logits"], ra["logits"][:, pi])
    assert np.array_equal(pi[rb["idx"]], ra["idx"])
    assert np.array_equal(rb["w"], ra["w"])
    # expert-major accumulation: the renaming reorders the fp64 sum of a
    # token's k expert outputs
    scale = np.abs(ra["y"]).max()
    assert np.abs(rb["y"] - ra["y"]).max() <= 1e-14 * scale


GPU_CASES = ORACLE_CASES + [
    CONFIGS["qwen3_decode"],
    small_cfg("int4_sym_g128", name="relabel_tiles96", T=1300, E=2, k=1, F=384),
    small_cfg("int4_asym_g128", name="relabel_prefill", T=1024, d=1024, E=8, k=2, F=640, S=1, Fs=384),
]


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", GPU_CASES, ids=lambda c: c.name + "_" + c.wformat)
def test_forward_expert_relabelling_invariance(cfg):
    import torch
    from quantized_mixture_experts_qmoe_amd import QMoE
    from gpu_util import to_dev_bf16

    print(f"[case] relabelled forward {cfg}", flush=True)
    inp = make_inputs(cfg, seed=11)
    pi = np.random.default_rng(5).permutation(cfg.E)
    T = cfg.T
    x = to_dev_bf16(inp.x)
    out = []
    for layer_inp in (inp, relabel(inp, pi)):
        layer = QMoE(layer_inp, max_tokens=T)
        route = QMoE.route_buffers(T, cfg.E, cfg.k)
        y = layer.forward(x, route=route)
        torch.cuda.synchronize()
        out.append((y.view(torch.int16).cpu().numpy().view(np.uint16), route["logits"].cpu().numpy(),
                    route["topk_idx"].cpu().numpy(), route["topk_w"].cpu().numpy()))
        del layer
    (ya, la, ia, wa), (yb, lb, ib, wb) = out
    s = np.sort(la, axis=1)
    assert (np.diff(s, axis=1) != 0).all(), "exact score ties: the renaming may reorder them"
    assert np.array_equal(lb, la[:, pi])
    assert np.array_equal(pi[ib], ia)
    assert np.array_equal(wb, wa)
    assert np.array_equal(yb, ya)
