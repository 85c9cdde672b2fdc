"""ctypes front end of the fp64 CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this module. The product path (the HIP library and its binding) never does.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmoe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FORMAT_CODES = {"int8_sym_ch": 0, "int4_asym_g128": 1, "int4_sym_g128": 2, "int3_sym_g128": 3,
                "fp8e4m3_ch": 4}
# router weight quantization per expert row (0: the weight as given)
ROUTER_QUANT_CODES = {"none": 0, "int8": 1, "fp8": 2}
GROUP_FORMATS = ("int4_asym_g128", "int4_sym_g128", "int3_sym_g128")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no fast-math, no contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        P = C.c_void_p
        L.orc_fp16_round.restype = C.c_float
        L.orc_fp16_round.argtypes = [C.c_float]
        L.orc_e4m3_decode.restype = C.c_double
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_e4m3_encode.argtypes = [C.c_float]
        L.orc_quantize.restype = C.c_int
        L.orc_quantize.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P]
        L.orc_dequantize.restype = C.c_int
        L.orc_dequantize.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P]
        L.orc_route_f32.restype = C.c_int
        L.orc_route_f32.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P]
        L.orc_dispatch.restype = C.c_int
        L.orc_dispatch.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, P]
        L.orc_layer_create.restype = P
        L.orc_layer_create.argtypes = [C.c_int] * 11 + [P, P, P, P, P, P, C.POINTER(C.c_int)]
        L.orc_layer_free.restype = None
        L.orc_layer_free.argtypes = [P]
        L.orc_layer_codes.restype = C.c_int
        L.orc_layer_codes.argtypes = [P, C.c_int, C.c_int, P, P, P]
        L.orc_forward.restype = C.c_int
        L.orc_forward.argtypes = [P, P, C.c_int, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def fp16_round(x: float) -> float:
    return lib().orc_fp16_round(float(x))


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(v: float) -> int:
    return int(lib().orc_e4m3_encode(float(v)))


def _nscales(fmt: str, N: int, K: int, group: int) -> int:
    return N * (K // group) if fmt in GROUP_FORMATS else N


def quantize(fmt: str, w: np.ndarray, group: int = 128):
    """Quantize w[N][K] -> (codes int8 [N][K], scale, zero) as the oracle does."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    q = np.zeros((N, K), np.int8)
    ns = _nscales(fmt, N, K, group)
    G = ns // N
    s = np.zeros((N, G), np.float32)
    z = np.zeros((N, G), np.float32)
    rc = lib().orc_quantize(FORMAT_CODES[fmt], N, K, group, _p(w), _p(q), _p(s), _p(z))
    if rc != 0:
        raise ValueError(f"orc_quantize rc={rc}")
    return q, s, z


def dequantize(fmt: str, q: np.ndarray, s: np.ndarray, z: np.ndarray, group: int = 128) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    N, K = q.shape
    out = np.zeros((N, K), np.float64)
    rc = lib().orc_dequantize(FORMAT_CODES[fmt], N, K, group, _p(q),
                              _p(np.ascontiguousarray(s, np.float32)), _p(np.ascontiguousarray(z, np.float32)),
                              _p(out))
    if rc != 0:
        raise ValueError(f"orc_dequantize rc={rc}")
    return out


def route(logits: np.ndarray, k: int, renorm: bool = True):
    """Top-k + softmax weights from fp32 logits [T][E] -> (idx int32, w f64, margin f64)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    m = np.zeros((T,), np.float64)
    rc = lib().orc_route_f32(T, E, k, int(renorm), _p(logits), _p(idx), _p(w), _p(m))
    if rc != 0:
        raise ValueError(f"orc_route_f32 rc={rc}")
    return idx, w, m


def dispatch(idx: np.ndarray, E: int):
    """Expert-centric task list -> (counts, offsets, perm, inv), all int32."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.zeros((E,), np.int32)
    offsets = np.zeros((E + 1,), np.int32)
    perm = np.zeros((T * k,), np.int32)
    inv = np.zeros((T * k,), np.int32)
    rc = lib().orc_dispatch(T, E, k, _p(idx), _p(counts), _p(offsets), _p(perm), _p(inv))
    if rc != 0:
        raise ValueError(f"orc_dispatch rc={rc}")
    return counts, offsets, perm, inv


class OracleLayer:
    """The oracle's own quantized copy of one layer (codes from the oracle quantizer)."""

    def __init__(self, inp):
        cfg = inp.cfg
        self.cfg = cfg
        n = cfg.E + cfg.S
        self._keep = [np.ascontiguousarray(a, np.float32) for a in inp.w_gate + inp.w_up + inp.w_down]
        arr = (C.c_void_p * n)
        wg = arr(*[a.ctypes.data for a in self._keep[0:n]])
        wu = arr(*[a.ctypes.data for a in self._keep[n:2 * n]])
        wd = arr(*[a.ctypes.data for a in self._keep[2 * n:3 * n]])
        wr = np.ascontiguousarray(inp.w_router)
        bias = None if inp.bias is None else np.ascontiguousarray(inp.bias, np.float32)
        fmts = None if cfg.expert_formats is None else np.array([FORMAT_CODES[f] for f in cfg.expert_formats],
                                                                  np.int32)
        err = C.c_int(0)
        self.h = lib().orc_layer_create(cfg.d, cfg.F, cfg.E, cfg.k, cfg.S, cfg.Fs, FORMAT_CODES[cfg.wformat],
                                        cfg.group, int(cfg.renormalize), int(cfg.router_fp32),
                                        ROUTER_QUANT_CODES[cfg.router_quant], _p(fmts), _p(wr), _p(bias),
                                        C.cast(wg, C.c_void_p), C.cast(wu, C.c_void_p), C.cast(wd, C.c_void_p),
                                        C.byref(err))
        self._keep = None   # the oracle holds its own codes now
        if not self.h:
            raise ValueError(f"orc_layer_create err={err.value}")

    def close(self):
        if getattr(self, "h", None):
            lib().orc_layer_free(self.h)
            self.h = None

    def __del__(self):
        self.close()

    def codes(self, expert: int, matrix: int):
        cfg = self.cfg
        f = cfg.F if expert < cfg.E else cfg.Fs
        N, K = (f, cfg.d) if matrix < 2 else (cfg.d, f)
        G = K // cfg.group if cfg.expert_format(expert) in GROUP_FORMATS else 1
        q = np.zeros((N, K), np.int8)
        s = np.zeros((N, G), np.float32)
        z = np.zeros((N, G), np.float32)
        rc = lib().orc_layer_codes(self.h, expert, matrix, _p(q), _p(s), _p(z))
        if rc != 0:
            raise ValueError("orc_layer_codes")
        return q, s, z

    def forward(self, x: np.ndarray, tokens: Optional[Sequence[int]] = None, given: Optional[np.ndarray] = None):
        """Returns dict(y, logits, idx, w, margin) for the listed tokens (all if None)."""
        cfg = self.cfg
        x = np.ascontiguousarray(x, np.uint16)
        T = x.shape[0]
        tok = None if tokens is None else np.ascontiguousarray(tokens, np.int32)
        n = T if tok is None else tok.shape[0]
        y = np.zeros((n, cfg.d), np.float64)
        lg = np.zeros((n, cfg.E), np.float64)
        idx = np.zeros((n, cfg.k), np.int32)
        w = np.zeros((n, cfg.k), np.float64)
        m = np.zeros((n,), np.float64)
        g = None if given is None else np.ascontiguousarray(given, np.int32)
        rc = lib().orc_forward(self.h, _p(x), n, _p(tok), _p(g), _p(y), _p(lg), _p(idx), _p(w), _p(m))
        if rc != 0:
            raise ValueError(f"orc_forward rc={rc}")
        return dict(y=y, logits=lg, idx=idx, w=w, margin=m)
