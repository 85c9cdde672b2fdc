"""Seeded synthetic workloads for the quantized top-k MoE layer.

This module only draws random tensors and names the layer shapes. It holds none
of the layer's arithmetic (no quantization, routing or expert math), so the HIP
library and the CPU oracle can both be fed from it without sharing any method
code.

Shapes follow the models the source pages measure: a Mixtral-style 8-expert
top-2 layer, Qwen3-30B-A3B (128 experts, top-8; pages: IT Donga article on
DREAM-MoE / SRA-MoE, experiment paragraphs), DeepSeek-V2-Lite (64 routed experts
top-6 plus 2 shared experts; same article, DREAM-MoE experiments) and a
decode-shaped batch of 16 tokens.  Real routers' load skew is imitated with a
per-expert logit bias drawn from N(0, 1) on the Qwen3 prefill shape.

Draw order (fixed, NumPy PCG64 ``default_rng(seed)``):
  1. router weight W_r [E][d]   ~ N(0, 0.02)  (rounded to bf16 unless router_fp32)
  2. router bias [E]            ~ N(0, 1)     (only where the config has one)
  3. for each routed expert, then each shared expert:
       W_gate [F][d], W_up [F][d], W_down [d][F]  ~ N(0, 0.02), fp32 pre-quant
  4. activations x [T][d]       ~ N(0, 1), rounded to bf16
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

# Weight format names, in the order of the C-ABI enum ``qmoe_wformat``.
WFORMATS = ("int8_sym_ch", "int4_asym_g128", "int4_sym_g128", "int3_sym_g128", "fp8e4m3_ch")


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens in the batch
    d: int            # d_model
    E: int            # routed experts
    k: int            # experts per token
    F: int            # d_ff of a routed expert
    wformat: str      # one of WFORMATS
    S: int = 0        # always-on shared experts
    Fs: int = 0       # d_ff of a shared expert
    router_fp32: bool = False
    router_quant: str = "none"   # router weight quantized per expert row: "none", "int8" or "fp8"
    # per-expert formats (E routed then S shared, each one of WFORMATS); None: all `wformat`
    expert_formats: Optional[Tuple[str, ...]] = None
    bias: bool = False
    renormalize: bool = True
    group: int = 128

    def expert_format(self, i: int) -> str:
        return self.wformat if self.expert_formats is None else self.expert_formats[i]

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.T * self.k

    def expert_flops(self) -> float:
        """Algorithmic FLOPs of one forward: the routed and shared SwiGLU experts
        (three d x F products each) plus the router product."""
        return (2.0 * self.T * self.k * 3 * self.d * self.F
                + 2.0 * self.T * self.S * 3 * self.d * self.Fs
                + 2.0 * self.T * self.d * self.E)


CONFIGS = {
    "tiny": LayerConfig("tiny", T=64, d=256, E=8, k=2, F=512, wformat="int8_sym_ch",
                        router_fp32=True),
    "mixtral_prefill": LayerConfig("mixtral_prefill", T=4096, d=4096, E=8, k=2, F=14336,
                                   wformat="int4_asym_g128"),
    "qwen3_prefill": LayerConfig("qwen3_prefill", T=8192, d=2048, E=128, k=8, F=768,
                                 wformat="int4_sym_g128", bias=True),
    "dsv2lite_prefill": LayerConfig("dsv2lite_prefill", T=2048, d=2048, E=64, k=6, F=1408,
                                    wformat="int3_sym_g128", S=2, Fs=1408),
    "qwen3_decode": LayerConfig("qwen3_decode", T=16, d=2048, E=128, k=8, F=768,
                                wformat="int4_sym_g128"),
    "qwen3_decode_fp8": LayerConfig("qwen3_decode_fp8", T=16, d=2048, E=128, k=8, F=768,
                                    wformat="fp8e4m3_ch"),
    # per-expert precision: one expert in eight (16 of 128) in INT8, the rest INT4
    "qwen3_prefill_mixed": LayerConfig("qwen3_prefill_mixed", T=8192, d=2048, E=128, k=8, F=768,
                                       wformat="int4_sym_g128", bias=True,
                                       expert_formats=tuple("int8_sym_ch" if e % 8 == 0 else "int4_sym_g128"
                                                            for e in range(128))),
    "qwen3_decode_mixed": LayerConfig("qwen3_decode_mixed", T=16, d=2048, E=128, k=8, F=768,
                                      wformat="int4_sym_g128",
                                      expert_formats=tuple("int8_sym_ch" if e % 8 == 0 else "int4_sym_g128"
                                                           for e in range(128))),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns as uint16."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    w_router: np.ndarray                 # [E][d] float32 if router_fp32 else uint16 (bf16 bits)
    bias: Optional[np.ndarray]           # [E] float32 or None
    w_gate: List[np.ndarray]             # E+S arrays [F][d] float32
    w_up: List[np.ndarray]               # E+S arrays [F][d] float32
    w_down: List[np.ndarray]             # E+S arrays [d][F] float32
    x: np.ndarray                        # [T][d] uint16 (bf16 bits)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def make_inputs(cfg: LayerConfig, seed: int = 0) -> LayerInputs:
    """Draw one layer's router, expert weights and activations in the fixed order."""
    rng = np.random.default_rng(seed)
    wr = _normal(rng, (cfg.E, cfg.d), 0.02)
    if not cfg.router_fp32:
        wr = f32_to_bf16_bits(wr)
    bias = _normal(rng, (cfg.E,), 1.0) if cfg.bias else None
    wg, wu, wd = [], [], []
    for i in range(cfg.E + cfg.S):
        f = cfg.F if i < cfg.E else cfg.Fs
        wg.append(_normal(rng, (f, cfg.d), 0.02))
        wu.append(_normal(rng, (f, cfg.d), 0.02))
        wd.append(_normal(rng, (cfg.d, f), 0.02))
    x = f32_to_bf16_bits(_normal(rng, (cfg.T, cfg.d), 1.0))
    return LayerInputs(cfg, wr, bias, wg, wu, wd, x)


def make_x(cfg: LayerConfig, T: int, seed: int) -> np.ndarray:
    """An independent batch of bf16 activations [T][d] (for multi-batch tests)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(_normal(rng, (T, cfg.d), 1.0))


def make_logits(T: int, E: int, seed: int, kind: str = "normal", k: int = 2) -> np.ndarray:
    """Synthetic fp32 router logits for routing-only tests.

    kind: "normal"  N(0, 1)
          "grid"    values on a 1/8 grid in [-1, 1] (many exact ties), with
                    +0.0 and -0.0 both present
          "equal"   every row constant (all experts tie)
          "hot"     one expert far above the rest for every token, others N(0,1)
          "sparse"  only experts 0..k win (every other expert gets no token)
    """
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if kind == "grid":
        a = (rng.integers(-8, 9, size=(T, E)).astype(np.float32) / np.float32(8.0))
        z = a == 0
        sign = rng.integers(0, 2, size=(T, E)).astype(bool)
        a[z & sign] = np.float32(-0.0)
        return a
    if kind == "equal":
        v = rng.standard_normal((T, 1), dtype=np.float32)
        return np.repeat(v, E, axis=1)
    if kind == "hot":
        a = rng.standard_normal((T, E), dtype=np.float32)
        hot = int(rng.integers(0, E))
        a[:, hot] = np.float32(100.0)
        return a
    if kind == "sparse":
        a = rng.standard_normal((T, E), dtype=np.float32) - np.float32(50.0)
        n = max(1, min(E, k + 1))
        a[:, :n] += np.float32(100.0)
        return a
    raise ValueError(kind)


@dataclasses.dataclass
class AtomicInputs:
    """Seeded synthetic atomic-expert layer (OmniMoE shapes): bf16 bit patterns."""
    router_rows: np.ndarray   # [n_rows][d]
    router_cols: np.ndarray   # [n_cols][d]
    w_in: np.ndarray          # [N][d]
    w_out: np.ndarray         # [N][d]
    x: np.ndarray             # [T][d]


def make_atomic_inputs(T: int, d: int, n_rows: int, n_cols: int, seed: int = 0) -> AtomicInputs:
    """Draw order: R_r, R_c, W, V ~ N(0, 0.02), then x ~ N(0, 1); all rounded to bf16."""
    rng = np.random.default_rng(seed)
    n = n_rows * n_cols

    def draw(shape, std):
        return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
    rr = draw((n_rows, d), 0.02)
    rc = draw((n_cols, d), 0.02)
    w_in = draw((n, d), 0.02)
    w_out = draw((n, d), 0.02)
    x = draw((T, d), 1.0)
    return AtomicInputs(rr, rc, w_in, w_out, x)
