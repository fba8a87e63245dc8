"""Seeded synthetic inputs for the sparse MoE experts layer.

This module only draws random numbers (see ``synth.c`` for the counter-based generator); it holds
none of the MoE method's arithmetic. Both the GPU path's tests/bench and the CPU oracle take their
inputs from here, so the same bytes reach both sides.

Workload recipes follow the five layer shapes this project is measured on (tiny fp32 check layer,
Mixtral-shaped prefill and decode, a skewed 128-expert layer, a DeepSeek-V3-shaped fine-grained FP8
layer). Seeds are ``1000*cfg + tau`` with tau = 0: x, 1: router logits or router weight,
2: W_gate, 3: W_up, 4: W_down. Standard deviations are ``1/sqrt(fan_in)`` for expert weights
(fan_in = d for gate/up, f for down), 0.02 for the router weight and 1 for x and logits.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``libsynth.so`` with gcc (host only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        u64, dbl, vp = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u64, u64, dbl, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, dbl, vp]
        lib.synth_skewed_logits.argtypes = [u64, u64, u64, dbl, vp]
        lib.synth_f32_to_bf16.argtypes = [vp, u64, vp]
        for fn in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_skewed_logits,
                   lib.synth_f32_to_bf16):
            fn.restype = None
        _lib = lib
    return _lib


def normal_f32(seed: int, shape, sigma: float = 1.0, first: int = 0) -> np.ndarray:
    """sigma * N(0,1) draws for element indices [first, first + prod(shape)), fp32."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(seed, first, n, float(sigma), out.ctypes.data)
    return out.reshape(shape)


def normal_bf16(seed: int, shape, sigma: float = 1.0, first: int = 0) -> np.ndarray:
    """Same draws as :func:`normal_f32`, rounded to bf16; returned as uint16 bit patterns."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(seed, first, n, float(sigma), out.ctypes.data)
    return out.reshape(shape)


def skewed_logits(seed: int, T: int, E: int, scale: float = 2.0) -> np.ndarray:
    """N(0,1) logits plus b_e = scale * ln(1/(e+1)) per expert (a Zipf-like load skew)."""
    out = np.empty(T * E, dtype=np.float32)
    _load().synth_skewed_logits(seed, T, E, float(scale), out.ctypes.data)
    return out.reshape(T, E)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(a.ctypes.data, a.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------------
# Layer workloads
# --------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class LayerSpec:
    """Shape and input recipe of one MoE layer workload.

    dtype: "f32" (everything fp32), "bf16" (bf16 x and weights), "fp8" (bf16 x, fp32 weight
    masters that the path quantises to e4m3 with 128x128 block scales).
    logits: "given" (N(0,1) logits, optionally skewed) or "router" (x . Wr^T with Wr ~ N(0, 0.02)).
    """

    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    dtype: str
    logits: str = "given"
    skew: float = 0.0
    seed_base: int = 0          # seeds = seed_base + tau
    x_seed: int | None = None   # overrides seed_base + 0 (decode reuses the prefill layer)

    @property
    def P(self) -> int:
        return self.T * self.k

    def seed(self, tau: int) -> int:
        if tau == 0 and self.x_seed is not None:
            return self.x_seed
        return self.seed_base + tau

    def with_(self, **kw) -> "LayerSpec":
        return replace(self, **kw)

    def active_flops(self) -> float:
        return 6.0 * self.P * self.d * self.f


# The five workloads. Names state what they are.
TINY_F32 = LayerSpec("tiny_f32_T64_d128_f256_E8_k2", 64, 128, 256, 8, 2, "f32", "given", 0.0, 1000)
MIXTRAL_PREFILL = LayerSpec("mixtral_prefill_bf16_T4096_d4096_f14336_E8_k2", 4096, 4096, 14336, 8, 2,
                            "bf16", "router", 0.0, 2000)
MIXTRAL_DECODE = LayerSpec("mixtral_decode_bf16_T32_d4096_f14336_E8_k2", 32, 4096, 14336, 8, 2,
                           "bf16", "router", 0.0, 2000, x_seed=3000)
SKEWED_128E = LayerSpec("skewed_bf16_T16384_d2048_f768_E128_k8", 16384, 2048, 768, 128, 8, "bf16",
                        "given", 2.0, 4000)
DSV3_FP8 = LayerSpec("dsv3_fp8_T8192_d7168_f2048_E256_k8", 8192, 7168, 2048, 256, 8, "fp8", "given",
                     0.0, 5000)

WORKLOADS = {s.name: s for s in (TINY_F32, MIXTRAL_PREFILL, MIXTRAL_DECODE, SKEWED_128E, DSV3_FP8)}


def gen_x(spec: LayerSpec) -> np.ndarray:
    """Token activations x [T, d]: fp32 for f32 layers, bf16 bits (uint16) otherwise."""
    if spec.dtype == "f32":
        return normal_f32(spec.seed(0), (spec.T, spec.d), 1.0)
    return normal_bf16(spec.seed(0), (spec.T, spec.d), 1.0)


def gen_logits(spec: LayerSpec) -> np.ndarray:
    """Given router logits [T, E] fp32 (only for logits == "given")."""
    assert spec.logits == "given"
    if spec.skew:
        return skewed_logits(spec.seed(1), spec.T, spec.E, spec.skew)
    return normal_f32(spec.seed(1), (spec.T, spec.E), 1.0)


def gen_router_weight(spec: LayerSpec) -> np.ndarray:
    """Router weight Wr [E, d] fp32, N(0, 0.02) (only for logits == "router")."""
    assert spec.logits == "router"
    return normal_f32(spec.seed(1), (spec.E, spec.d), 0.02)


def _w_sigma(which: str, spec: LayerSpec) -> float:
    return 1.0 / math.sqrt(spec.d if which in ("gate", "up") else spec.f)


def _w_shape(which: str, spec: LayerSpec):
    return (spec.f, spec.d) if which in ("gate", "up") else (spec.d, spec.f)


_TAU = {"gate": 2, "up": 3, "down": 4}


def gen_expert_weight(spec: LayerSpec, which: str, experts=None) -> np.ndarray:
    """Expert weight W_gate/W_up [E, f, d] or W_down [E, d, f] (nn.Linear layout, y = x W^T).

    f32 layers: fp32. bf16 layers: bf16 bits. fp8 layers: the fp32 masters (quantised later).
    ``experts`` selects a subset (list of expert ids) with the same bytes as the full draw.
    """
    rows, cols = _w_shape(which, spec)
    sig = _w_sigma(which, spec)
    seed = spec.seed(_TAU[which])
    ids = range(spec.E) if experts is None else list(experts)
    per = rows * cols
    fn = normal_bf16 if spec.dtype == "bf16" else normal_f32
    dt = np.uint16 if spec.dtype == "bf16" else np.float32
    out = np.empty((len(ids), rows, cols), dtype=dt)
    for n, e in enumerate(ids):
        out[n] = fn(seed, (rows, cols), sig, first=e * per)
    return out
