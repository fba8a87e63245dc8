"""Helpers for the GPU parity tests: host <-> device copies, cached workload inputs, the
tolerance check. Inputs come from ``synth``; expected values only from ``oracle``."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import synth

DEV = "cuda"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    a = to_host(t)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def assert_close_rel_max(got: np.ndarray, ref: np.ndarray, rel: float, what: str = ""):
    """max |got - ref| <= rel * max |ref| over all elements."""
    err = np.abs(got - ref).max()
    scale = np.abs(ref).max()
    log("%s max|err| = %.3e, max|ref| = %.3e, ratio = %.3e (bound %.1e)"
        % (what, err, scale, err / scale, rel))
    assert err <= rel * scale, (what, err, scale)


@functools.lru_cache(maxsize=4)
def layer_inputs(spec: synth.LayerSpec):
    """Host arrays for a workload (bf16 as uint16 bits, fp8 layers as fp32 masters)."""
    d = dict(x=synth.gen_x(spec))
    if spec.logits == "given":
        d["logits"] = synth.gen_logits(spec)
    else:
        d["Wr"] = synth.gen_router_weight(spec)
    for n in ("gate", "up", "down"):
        d["W" + n] = synth.gen_expert_weight(spec, n)
    return d


def oracle_experts(spec, inp):
    return oracle.Experts(inp["Wgate"], inp["Wup"], inp["Wdown"])
