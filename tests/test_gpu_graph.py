"""A forward recorded once into a HIP graph and replayed: every replay equals
an eager call on the same input bit for bit (qmoe_forward issues only kernel
launches and, for requested routing outputs, device copies on the caller's
stream, and allocates nothing per call, so a capturing caller can record it).
Between replays the test rewrites the input and runs eager forwards of its
own, so each replay is checked against fresh state."""
import numpy as np
import pytest
import torch

import quantized_mixture_experts_qmoe_amd as Q
from quantized_mixture_experts_qmoe_amd.inputs import CONFIGS, LayerConfig, make_inputs, make_x
from gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu


def capture(fn):
    """Records fn() into a torch CUDA graph (captured on torch's side stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("cfg", [
    # decode tiles, one-workgroup top-k + dispatch
    CONFIGS["qwen3_decode"],
    # prefill tiles: gating in the router's epilogue, fused row sums
    LayerConfig("graph_prefill", T=700, d=1024, E=16, k=2, F=1024, wformat="int4_sym_g128"),
    # shared expert, fp32 router with the separate row-sum kernel
    LayerConfig("graph_asym_shared", T=200, d=512, E=8, k=2, F=512, wformat="int4_asym_g128", S=1, Fs=512,
                router_fp32=True),
], ids=lambda c: c.name)
@pytest.mark.parametrize("entry", ["forward", "forward_static"])
def test_graph_replay_equals_eager(cfg, entry):
    inp = make_inputs(cfg, seed=5)
    layer = Q.QMoE(inp, max_tokens=cfg.T)
    fn_c = Q.qmoe_forward if entry == "forward" else Q.qmoe_forward_static
    try:
        x = to_dev_bf16(inp.x)
        y = torch.empty_like(x)
        route = Q.QMoE.route_buffers(cfg.T, cfg.E, cfg.k)
        names = ("logits", "topk_idx", "topk_w", "counts", "offsets", "perm")
        dbg = Q.QmoeRouteOut(*[route[n].data_ptr() for n in names])

        def call():
            rc = fn_c(layer.ctx, x.data_ptr(), cfg.T, y.data_ptr(), dbg, torch.cuda.current_stream().cuda_stream)
            assert rc == Q.QMOE_OK, (rc, Q.qmoe_last_error())

        print(f"[case] graph capture {cfg.name} {entry}", flush=True)
        g = capture(call)
        for rep in range(3):
            x.copy_(to_dev_bf16(make_x(cfg, cfg.T, seed=100 + rep)))
            y.fill_(float("nan"))
            torch.cuda.synchronize()
            print(f"[case] graph replay {cfg.name} {entry} #{rep}", flush=True)
            g.replay()
            torch.cuda.synchronize()
            y_g = y.clone()
            r_g = {n: route[n].clone() for n in names}
            # the eager call on the same input (its own launches, same workspace)
            y_e = layer.forward(x, route=(r_e := Q.QMoE.route_buffers(cfg.T, cfg.E, cfg.k)))
            torch.cuda.synchronize()
            assert torch.equal(y_g.view(torch.int16), y_e.view(torch.int16)), (cfg.name, entry, rep)
            for n in names:
                assert torch.equal(r_g[n], r_e[n]), (cfg.name, entry, rep, n)
            assert not torch.isnan(y_g.float()).any()
        del g
    finally:
        torch.cuda.synchronize()
        layer.close()
