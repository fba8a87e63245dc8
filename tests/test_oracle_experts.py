"""Pins for the oracle's experts and weighted combine.

Layer definition: Transformers "Experts backends" page, intro (all backends compute the same
function: pick k experts per token, project through their parameters, combine with the routing
weights); the gated-MLP/SwiGLU expert from the rows deepgemm_megamoe and sonicmoe of its backends
table. The independent check here is the dense formulation (run every expert on every token with
numpy matmuls, then mask by routing), which no backend on the pages uses, plus closed forms.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "swiglu_worked_example.txt")


def _parse_golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, rhs = [p.strip() for p in line.split("=")]
        rows = [[float(v) for v in r.split()] for r in rhs.split(";")]
        vals[key] = np.array(rows if len(rows) > 1 else rows[0], np.float64)
    return vals


def _dense_reference(xf, Wg, Wu, Wd, ids, w):
    """Every expert on every token, masked by the routing weights (fp64 numpy)."""
    T = xf.shape[0]
    E, f, d = Wg.shape
    out = np.zeros((T, d), np.float64)
    for e in range(E):
        g = xf @ Wg[e].T
        u = xf @ Wu[e].T
        h = g / (1.0 + np.exp(-g)) * u
        y = h @ Wd[e].T
        m = np.zeros(T)
        for j in range(ids.shape[1]):
            m += np.where(ids[:, j] == e, w[:, j].astype(np.float64), 0.0)
        out += m[:, None] * y
    return out


def _weights_f64(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else \
        a.astype(np.float64)


def test_swiglu_worked_example():
    g = _parse_golden()
    x = g["x"].astype(np.float32)[None, :]
    Wg = g["W_gate"].astype(np.float32)[None]
    Wu = g["W_up"].astype(np.float32)[None]
    Wd = g["W_down"].astype(np.float32)[None]
    ex = oracle.Experts(Wg, Wu, Wd)
    h, y = oracle.expert_pairs(x, ex, np.array([0]), np.array([0]))
    np.testing.assert_allclose(h[0], g["h"], rtol=1e-15)
    np.testing.assert_allclose(y[0], g["y"], rtol=1e-15)
    # k = 1 with one expert: the layer output is that expert's output (weight exactly 1)
    ids, w = oracle.route(np.zeros((1, 1), np.float32), 1)
    out = oracle.moe_forward(x, ex, ids, w)
    np.testing.assert_allclose(out[0], g["y"], rtol=1e-15)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_is_textbook_swiglu_mlp(dtype):
    spec = synth.TINY_F32.with_(E=1, k=1, T=16, dtype=dtype)
    x = synth.gen_x(spec)
    Wg, Wu, Wd = (synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down"))
    ex = oracle.Experts(Wg, Wu, Wd)
    ids = np.zeros((16, 1), np.int32)
    w = np.ones((16, 1), np.float32)
    out = oracle.moe_forward(x, ex, ids, w)
    xf = _weights_f64(x)
    g = xf @ _weights_f64(Wg[0]).T
    u = xf @ _weights_f64(Wu[0]).T
    ref = (g * (1.0 / (1.0 + np.exp(-g))) * u) @ _weights_f64(Wd[0]).T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("spec", [
    synth.TINY_F32,
    synth.TINY_F32.with_(dtype="bf16", T=40, d=64, f=192, E=6, k=3),
    synth.SKEWED_128E.with_(T=96, d=64, f=128, E=16, k=4),
], ids=["tiny_f32", "bf16_E6_k3", "skewed_E16_k4"])
def test_matches_dense_formulation(spec):
    x = synth.gen_x(spec)
    Wg, Wu, Wd = (synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down"))
    ex = oracle.Experts(Wg, Wu, Wd)
    logits = synth.gen_logits(spec)
    ids, w = oracle.route(logits, spec.k)
    out = oracle.moe_forward(x, ex, ids, w)
    ref = _dense_reference(_weights_f64(x), _weights_f64(Wg), _weights_f64(Wu), _weights_f64(Wd),
                           ids, w)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    # a token subset gives the same rows
    sub = np.array([5, 0, spec.T - 1], np.int32)
    np.testing.assert_array_equal(oracle.moe_forward(x, ex, ids, w, tokens=sub), out[sub])


def test_identical_experts_make_routing_irrelevant():
    spec = synth.TINY_F32.with_(T=24)
    x = synth.gen_x(spec)
    one = [synth.gen_expert_weight(spec.with_(E=1), n) for n in ("gate", "up", "down")]
    ex = oracle.Experts(*[np.repeat(a, 8, axis=0) for a in one])
    ids, w = oracle.route(synth.gen_logits(spec), 2)
    out = oracle.moe_forward(x, ex, ids, w)
    single = oracle.moe_forward(x, oracle.Experts(*one), np.zeros((24, 1), np.int32),
                                np.ones((24, 1), np.float32))
    np.testing.assert_allclose(out, single, rtol=1e-6, atol=1e-7)  # sum of w is 1 to fp32 ulps


def test_token_permutation_equivariance():
    spec = synth.TINY_F32
    x = synth.gen_x(spec)
    ex = oracle.Experts(*(synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down")))
    logits = synth.gen_logits(spec)
    perm = np.random.default_rng(0).permutation(spec.T)
    ids, w = oracle.route(logits, 2)
    ids_p, w_p = oracle.route(logits[perm], 2)
    np.testing.assert_array_equal(
        oracle.moe_forward(x[perm], ex, ids_p, w_p), oracle.moe_forward(x, ex, ids, w)[perm])


def test_unfused_combine_equals_layer():
    spec = synth.TINY_F32.with_(k=3)
    x = synth.gen_x(spec)
    ex = oracle.Experts(*(synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down")))
    ids, w = oracle.route(synth.gen_logits(spec), 3)
    counts, offsets, sp, pp = oracle.permute(ids, spec.E)
    tok = sp // 3
    exp_of = ids.reshape(-1)[sp]
    _, y = oracle.expert_pairs(x, ex, tok, exp_of, want_h=False)
    out = oracle.combine_permuted(y, pp, w)
    np.testing.assert_allclose(out, oracle.moe_forward(x, ex, ids, w), rtol=1e-13, atol=1e-13)


def test_unused_experts_do_not_matter():
    # Experts that receive no token can hold anything (here NaN) without touching the output.
    spec = synth.SKEWED_128E.with_(T=64, d=64, f=128, E=32, k=2)
    x = synth.gen_x(spec)
    W = [synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down")]
    ids, w = oracle.route(synth.gen_logits(spec), 2)
    counts, *_ = oracle.permute(ids, spec.E)
    empty = np.flatnonzero(counts == 0)
    assert empty.size > 0
    out = oracle.moe_forward(x, oracle.Experts(*W), ids, w)
    for a in W:
        a[empty] = 0x7FC0  # bf16 NaN
    out2 = oracle.moe_forward(x, oracle.Experts(*W), ids, w)
    np.testing.assert_array_equal(out, out2)
