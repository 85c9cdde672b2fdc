"""The device quantizer (qmoe_pack_experts_device) against the host one: the
same bf16 expert weights, packed on the GPU from device memory and on the host
from their fp32 values, give bit-identical codes, scales and zeros and
bit-identical layer outputs; degenerate groups and rows (all zeros, negative
zeros) and fp16 scale saturation included. Plus the packing rate on a
Mixtral-shaped expert."""
import time

import numpy as np
import pytest
import torch

from quantized_mixture_experts_qmoe_amd import QMoE
from quantized_mixture_experts_qmoe_amd.inputs import LayerConfig, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs
from gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu

FORMATS = ["int8_sym_ch", "int4_asym_g128", "int4_sym_g128", "int3_sym_g128", "fp8e4m3_ch"]


def bf16_pair(a):
    """(bf16-valued fp32 host array, bf16 CUDA tensor) of the same values."""
    bits = f32_to_bf16_bits(a)
    return bf16_bits_to_f32(bits), torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def with_edge_cases(w, rng):
    w = w.copy()
    w[3, :] = 0.0                     # an all-zero row (every group of it)
    w[5, 128:256] = -0.0              # an all-negative-zero group
    w[6, 0:128] = 0.0
    w[6, 7] = -0.0
    w[9, 256:384] *= 1e8              # group scales past the fp16 range saturate
    return w


@pytest.mark.parametrize("fmt", FORMATS + ["mixed"])
def test_device_pack_equals_host_pack(fmt):
    mixed = fmt == "mixed"
    fm = tuple(FORMATS[(2 * e + 1) % 5] for e in range(5)) + ("int4_asym_g128",) if mixed else None
    cfg = LayerConfig(name=f"devpack_{fmt}", T=48, d=512, E=5, k=2, F=384, S=1, Fs=256,
                      wformat="int4_sym_g128" if mixed else fmt, expert_formats=fm, bias=True)
    print(f"[case] device pack {fmt}", flush=True)
    inp = make_inputs(cfg, seed=21)
    rng = np.random.default_rng(3)
    dev = ([], [], [])
    for lst, dl in ((inp.w_gate, dev[0]), (inp.w_up, dev[1]), (inp.w_down, dev[2])):
        for i in range(len(lst)):
            host_vals, t = bf16_pair(with_edge_cases(lst[i], rng))
            lst[i] = host_vals
            dl.append(t)
    host = QMoE(inp, max_tokens=cfg.T)
    devl = QMoE(inp, max_tokens=cfg.T, device_weights=dev)
    for e in range(cfg.E + cfg.S):
        for m in range(3):
            a, b = host.export(e, m), devl.export(e, m)
            for u, v, what in zip(a, b, ("codes", "scales", "zeros")):
                assert np.array_equal(u, v), (fmt, e, m, what)
    x = to_dev_bf16(inp.x)
    y1 = host.forward(x)
    y2 = devl.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), fmt
    host.close()
    devl.close()


def test_device_pack_rate():
    """Two Mixtral-shaped experts (d = 4096, d_ff = 14336, INT4 asym): the
    bf16 weights read once from HBM and the packed arena written once."""
    cfg = LayerConfig(name="devpack_rate", T=16, d=4096, E=2, k=1, F=14336, wformat="int4_asym_g128")
    inp = make_inputs(cfg, seed=5)
    dev = tuple([bf16_pair(w)[1] for w in ws] for ws in (inp.w_gate, inp.w_up, inp.w_down))
    QMoE(inp, max_tokens=16, device_weights=dev).close()   # warm-up (code objects, allocator)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    layer = QMoE(inp, max_tokens=16, device_weights=dev)
    t1 = time.perf_counter()
    layer.close()
    t2 = time.perf_counter()
    QMoE(inp, max_tokens=16).close()
    t3 = time.perf_counter()
    nbytes = sum(w.numel() * 2 for ws in dev for w in ws)
    print(f"[pack] 2 Mixtral-shaped INT4-asym experts ({nbytes / 1e6:.0f} MB of bf16): device quantizer "
          f"{(t1 - t0) * 1e3:.1f} ms ({nbytes / (t1 - t0) / 1e9:.0f} GB/s of bf16 input, allocation and workspace "
          f"included), host quantizer {(t3 - t2) * 1e3:.0f} ms", flush=True)
