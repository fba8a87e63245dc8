"""The oracle's precision against the fp32 per-token loop.

The layer's stated oracle is a plain per-token loop over the selected experts in fp32 (the
"eager" row of the Transformers "Experts backends" backends table: iterate the selected experts,
project their tokens, combine with the routing weights). ``oracle.moe_forward`` runs that loop with
every sum in fp64 and rounds nowhere, so it is closer to the exact result; ``oracle.moe_forward_f32``
is the same loop in fp32. These tests pin that the two agree far inside the layer tolerances
(max|err| <= 2e-2 * max|ref| for bf16 layers, 1e-4 * max|ref| internally for the fp32 layer), at
the real reduction lengths of the Mixtral-shaped layer (d = 4096, f = 14336), so comparing the GPU
with the fp64 loop is at least as strict as comparing it with the fp32 one.
"""
import numpy as np

import oracle
import synth


def _rel_max(a, b):
    return np.abs(np.asarray(a, np.float64) - b).max() / np.abs(b).max()


def test_tiny_fp32_loop_matches_fp64_loop():
    spec = synth.TINY_F32
    x, lg = synth.gen_x(spec), synth.gen_logits(spec)
    ex = oracle.Experts(*(synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down")))
    ids, w = oracle.route(lg, spec.k)
    r64 = oracle.moe_forward(x, ex, ids, w)
    r32 = oracle.moe_forward_f32(x, ex, ids, w)
    # fp32 sums of 128 and 256 terms: relative error ~1e-7 per output, far below 1e-4
    assert _rel_max(r32, r64) <= 5e-6


def test_mixtral_sized_fp32_loop_matches_fp64_loop():
    # the Mixtral-shaped reduction lengths (d = 4096, f = 14336) on two experts and four tokens
    spec = synth.MIXTRAL_DECODE.with_(name="mixtral_shape_T4_E2", T=4, E=2)
    x = synth.gen_x(spec)
    ex = oracle.Experts(*(synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down")))
    ids = np.array([[0, 1], [1, 0], [0, 1], [1, 0]], np.int32)
    w = np.array([[0.75, 0.25], [0.6, 0.4], [0.5, 0.5], [0.9, 0.1]], np.float32)
    r64 = oracle.moe_forward(x, ex, ids, w)
    r32 = oracle.moe_forward_f32(x, ex, ids, w)
    err = _rel_max(r32, r64)
    # sequential fp32 sums of 4096 and 14336 terms: ~sqrt(n) * 2^-24 relative, i.e. ~1e-5
    assert err <= 2e-4, err          # 100x inside the bf16 layer bound of 2e-2


def test_router_logits_fp32_sum_and_near_ties():
    # The Mixtral-shaped router (d = 4096, Wr ~ N(0, 0.02)): an fp32 sum in ascending order
    # differs from the fp64 sum by ~1e-6; the top-2 selections then differ only where the
    # fp64 logits are that close to a tie.
    spec = synth.MIXTRAL_PREFILL
    x, Wr = synth.gen_x(spec), synth.gen_router_weight(spec)
    l64 = oracle.router_logits(x, Wr)
    l32 = oracle.router_logits_f32(x, Wr)
    diff = np.abs(l32.astype(np.float64) - l64)
    assert diff.max() <= 1e-5 * (1.0 + np.abs(l64).max()), diff.max()
    ids64, _ = oracle.route(l64, spec.k)
    ids32, _ = oracle.route(l32, spec.k)
    flips = np.nonzero((ids64 != ids32).any(1))[0]
    srt = -np.sort(-l64.astype(np.float64), axis=1)
    margin = np.min(srt[:, :spec.k] - srt[:, 1:spec.k + 1], axis=1)   # closest adjacent pair
    assert np.all(margin[flips] <= 2 * diff.max()), (flips, margin[flips])
    assert flips.size <= 4, flips
