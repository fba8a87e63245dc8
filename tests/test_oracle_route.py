"""Pins for the oracle's router: softmax -> top-k -> renormalise.

Routing steps: lira-now "Mixture of Experts" explainer, section 5 (router step by step) and its
pseudocode; gyaansetu explainer, router top-k. Checks here do not re-type the oracle's formula:
they use hand-worked closed forms, brute force over all expert subsets, scipy's softmax and
invariants.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_worked_examples.txt")


def _golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, k, lg, ids, ws = [p.strip() for p in line.split("|")]
        if lg.startswith("raw:"):
            logits = [float(v) for v in lg[4:].split()]
        else:
            logits = [math.log(float(v)) for v in lg.split()]
        cases.append((name, int(k), logits, [int(i) for i in ids.split()],
                      [float(Fraction(w)) for w in ws.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c[0])
def test_worked_examples(case):
    name, k, logits, ids_ref, w_ref = case
    ids, w = oracle.route(np.array([logits], np.float32), k)
    assert ids[0].tolist() == ids_ref
    np.testing.assert_allclose(w[0], w_ref, rtol=2e-7, atol=0)


def _brute_force_topk(logits_row, k):
    """The k-subset of experts with the largest total softmax probability; among equal totals the
    lexicographically smallest index set; then ordered by probability (ties: lower index)."""
    p = softmax(logits_row.astype(np.float64))
    E = len(p)
    best, best_sum = None, -1.0
    for sub in itertools.combinations(range(E), k):
        s = sum(p[i] for i in sub)
        if s > best_sum * (1 + 1e-15):
            best, best_sum = sub, s
    order = sorted(best, key=lambda i: (-logits_row[i], i))
    return order, p


@pytest.mark.parametrize("k", [1, 2, 3])
def test_brute_force_tiny(k):
    logits = synth.normal_f32(1001, (64, 8))
    ids, w = oracle.route(logits, k)
    for t in range(64):
        order, p = _brute_force_topk(logits[t], k)
        assert ids[t].tolist() == order
        ref = p[order] / p[order].sum()
        np.testing.assert_allclose(w[t], ref, rtol=1e-6)


def test_invariants_many_experts():
    logits = synth.skewed_logits(4001, 512, 128, 2.0)
    k = 8
    ids, w = oracle.route(logits, k)
    # distinct ids in range
    assert ids.min() >= 0 and ids.max() < 128
    assert all(len(set(r)) == k for r in ids.tolist())
    # weights sum to 1 (within k ulps of fp32), descending, positive
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=k * 2 ** -23)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.all(w > 0)
    # selected logits are the k largest: no unselected logit exceeds the smallest selected one
    for t in range(512):
        sel = logits[t, ids[t]]
        rest = np.delete(logits[t], ids[t])
        assert rest.max() <= sel.min()


def test_k_equals_E_is_full_softmax():
    logits = synth.normal_f32(1002, (32, 16))
    ids, w = oracle.route(logits, 16)
    for t in range(32):
        order = sorted(range(16), key=lambda i: (-logits[t, i], i))
        assert ids[t].tolist() == order
        np.testing.assert_allclose(w[t], softmax(logits[t].astype(np.float64))[order], rtol=1e-6)


def test_k1_weight_exactly_one():
    logits = synth.normal_f32(1003, (100, 8))
    ids, w = oracle.route(logits, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(logits, axis=1))  # argmax returns first max


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_all_equal_logits(k):
    logits = np.full((5, 8), 0.25, np.float32)
    ids, w = oracle.route(logits, k)
    assert np.all(ids == np.arange(k))
    assert np.all(w == np.float32(1.0 / k))


def test_selection_uses_logits_not_rounded_probabilities():
    # Two logits one fp32 ulp apart: their exp() values may round together in fp32, but the
    # logit order is exact. The larger logit must be picked first.
    a = np.float32(-30.0)
    b = np.nextafter(a, np.float32(0))
    logits = np.array([[a, b, np.float32(-1e3), np.float32(-1e3)]], np.float32)
    ids, _ = oracle.route(logits, 1)
    assert ids[0, 0] == 1


def test_router_logits_match_dense_matmul():
    T, d, E = 16, 256, 8
    x = synth.normal_bf16(1100, (T, d))
    Wr = synth.normal_f32(1101, (E, d), 0.02)
    got = oracle.router_logits(x, Wr)
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ Wr.astype(np.float64).T
    np.testing.assert_allclose(got, ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    xf = synth.normal_f32(1102, (T, d))
    np.testing.assert_allclose(oracle.router_logits(xf, Wr),
                               xf.astype(np.float64) @ Wr.astype(np.float64).T, rtol=1e-6,
                               atol=1e-7)
