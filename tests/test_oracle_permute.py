"""Pins for the oracle's grouping of (token, slot) pairs by expert.

Transformers "Experts backends" page, backends table row grouped_mm: tokens are sorted by their
selected expert so one grouped GEMM covers all of them. Within an expert the order is the flat
pair index t*k + j (a stable sort; reading of a point the page leaves open).
"""
import numpy as np
import pytest

import oracle
import synth


def _check(ids, E):
    T, k = ids.shape
    P = T * k
    counts, offsets, sp, pp = oracle.permute(ids, E)
    flat = ids.reshape(-1)
    # counts: brute-force recount; sum = T*k
    assert np.array_equal(counts, np.array([np.sum(flat == e) for e in range(E)]))
    assert counts.sum() == P
    # offsets: exclusive scan, monotone, ends at P
    assert offsets[0] == 0 and offsets[-1] == P
    assert np.all(np.diff(offsets) == counts)
    # sorted_pair: a bijection on [0, P), equal to numpy's stable argsort by expert
    assert np.array_equal(np.sort(sp), np.arange(P))
    assert np.array_equal(sp, np.argsort(flat, kind="stable"))
    # experts non-decreasing along the sorted order; stable inside each group
    assert np.all(np.diff(flat[sp]) >= 0)
    for e in range(E):
        grp = sp[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(grp) > 0)
        assert np.all(flat[grp] == e)
    # pair_pos is the inverse permutation
    assert np.array_equal(pp[sp], np.arange(P))
    assert np.array_equal(sp[pp], np.arange(P))
    return counts


def test_tiny_uniform():
    ids, _ = oracle.route(synth.normal_f32(1001, (64, 8)), 2)
    _check(ids, 8)


def test_skewed_has_empty_groups():
    ids, _ = oracle.route(synth.skewed_logits(4001, 2048, 128, 2.0), 8)
    counts = _check(ids, 128)
    assert counts[0] == 2048          # expert 0 gets every token under this skew
    assert np.sum(counts == 0) > 0    # and some experts get none


def test_many_experts():
    ids, _ = oracle.route(synth.normal_f32(5001, (300, 256)), 8)
    _check(ids, 256)


def test_all_tokens_one_expert_and_single_token():
    ids = np.zeros((7, 1), np.int32)
    counts = _check(ids, 4)
    assert counts.tolist() == [7, 0, 0, 0]
    _check(np.array([[3, 1]], np.int32), 4)


def test_hand_example():
    # ids (T=3, k=2): pairs p = 0..5 -> experts 2,0,1,2,0,1
    ids = np.array([[2, 0], [1, 2], [0, 1]], np.int32)
    counts, offsets, sp, pp = oracle.permute(ids, 3)
    assert counts.tolist() == [2, 2, 2]
    assert offsets.tolist() == [0, 2, 4, 6]
    assert sp.tolist() == [1, 4, 2, 5, 0, 3]
    assert pp.tolist() == [4, 0, 2, 5, 1, 3]
