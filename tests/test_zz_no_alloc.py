"""qmoe_forward_static (the allocation-free forward, workspace in the library's
static per-device scratch) against qmoe_forward, through the C ABI: the same
layer, two calls in a row with the second batch smaller, outputs and routing
bit for bit equal. Also: a batch whose workspace does not fit is rejected."""
import ctypes as C

import numpy as np
import pytest
import torch

import quantized_mixture_experts_qmoe_amd as Q
from quantized_mixture_experts_qmoe_amd.inputs import CONFIGS, LayerConfig, make_inputs, make_x
from gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu

ROUTE_NAMES = ("logits", "topk_idx", "topk_w", "counts", "offsets", "perm")


def run_entry(fn, layer, x, T, E, k):
    """One call of a forward entry point with raw pointers; returns y and the routing."""
    y = torch.full_like(x, float("nan"))
    route = Q.QMoE.route_buffers(T, E, k)
    dbg = Q.QmoeRouteOut(*[route[n].data_ptr() for n in ROUTE_NAMES])
    stream = torch.cuda.current_stream().cuda_stream
    rc = fn(layer.ctx, x.data_ptr(), T, y.data_ptr(), dbg, stream)
    assert rc == Q.QMOE_OK, (rc, Q.qmoe_last_error())
    torch.cuda.synchronize()
    return y, route


@pytest.mark.parametrize("cfg", [
    # decode-shaped: one-workgroup top-k + dispatch, 16-row decode tiles
    CONFIGS["qwen3_decode"],
    # prefill-shaped: the multi-kernel dispatch and 64-row prefill tiles
    LayerConfig("static_prefill", T=300, d=1024, E=8, k=2, F=2048, wformat="int4_asym_g128"),
    # shared experts, INT3 and 64 experts
    LayerConfig("static_shared", T=160, d=512, E=64, k=6, F=256, wformat="int3_sym_g128", S=2, Fs=256),
], ids=lambda c: c.name)
def test_static_forward_equals_forward(cfg):
    inp = make_inputs(cfg, seed=3)
    layer = Q.QMoE(inp, max_tokens=cfg.T)
    try:
        sizes = (cfg.T, max(1, cfg.T // 4 + 1))   # the second call smaller
        for i, T in enumerate(sizes):
            bits = inp.x[:T] if i == 0 else make_x(cfg, T, seed=40 + i)
            x = to_dev_bf16(bits)
            print(f"[case] static forward {cfg.name} call {i} T={T}", flush=True)
            y_ref, r_ref = run_entry(Q.qmoe_forward, layer, x, T, cfg.E, cfg.k)
            y_st, r_st = run_entry(Q.qmoe_forward_static, layer, x, T, cfg.E, cfg.k)
            assert torch.equal(y_st.view(torch.int16), y_ref.view(torch.int16)), (cfg.name, T)
            for n in ROUTE_NAMES:
                assert torch.equal(r_st[n], r_ref[n]), (cfg.name, T, n)
    finally:
        layer.close()


def test_static_forward_rejects_a_batch_past_the_scratch():
    cfg = CONFIGS["qwen3_decode"].replace(name="static_big", T=1024)
    inp = make_inputs(cfg.replace(T=1), seed=0)
    layer = Q.QMoE(inp, max_tokens=cfg.T)
    try:
        x = torch.zeros((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
        y = torch.empty_like(x)
        rc = Q.qmoe_forward_static(layer.ctx, x.data_ptr(), cfg.T, y.data_ptr(), None,
                                   torch.cuda.current_stream().cuda_stream)
        assert rc == Q.QMOE_EUNSUPPORTED and "static scratch" in Q.qmoe_last_error()
        # T = 0 is a no-op, T past max_tokens is an argument error
        assert Q.qmoe_forward_static(layer.ctx, x.data_ptr(), 0, y.data_ptr(), None, None) == Q.QMOE_OK
        assert Q.qmoe_forward_static(layer.ctx, x.data_ptr(), cfg.T + 1, y.data_ptr(), None,
                                     None) == Q.QMOE_EINVAL
    finally:
        layer.close()
