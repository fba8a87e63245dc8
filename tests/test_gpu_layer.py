"""GPU parity of the whole layer (route -> permute -> grouped gated-MLP GEMMs -> combine) against
the oracle, through the C ABI.

Bounds (max over all compared output elements): bf16 layers max|err| <= 2e-2 * max|ref|;
the fp32 layer <= 1e-4 * max|ref| (fp32 end to end). Routing ids are bit-exact. Small shapes are
compared in full; the full-size workloads in the launch configuration the benchmark times are
compared on sampled tokens (the oracle computes them one by one).
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_softmax_amd as moe
import oracle
import synth
from gpu_util import (assert_close_rel_max, layer_inputs, log, out_to_f64, to_dev, to_host)

pytestmark = pytest.mark.gpu


def _run_gpu(spec, inp, y_layout="slots"):
    dev = {k: to_dev(v) for k, v in inp.items()}
    res = moe.moe_layer(dev["x"], dev["Wgate"], dev["Wup"], dev["Wdown"], spec.k,
                        logits=dev.get("logits"), w_router=dev.get("Wr"), y_layout=y_layout)
    torch.cuda.synchronize()
    return res


def _check_layer(spec, inp, res, rel, tokens=None):
    if "logits" in inp:
        lg = inp["logits"]
    else:
        lg = to_host(res.logits)  # the selection is replayed on the device's logits
        np.testing.assert_allclose(lg, oracle.router_logits(inp["x"], inp["Wr"]), rtol=0,
                                   atol=1e-4)
    ids_ref, w_ref = oracle.route(lg, spec.k)
    np.testing.assert_array_equal(to_host(res.topk_ids), ids_ref)
    np.testing.assert_allclose(to_host(res.topk_w), w_ref, rtol=0, atol=4e-7)
    counts, offsets, sp, pp = oracle.permute(ids_ref, spec.E)
    np.testing.assert_array_equal(to_host(res.perm.offsets), offsets)
    np.testing.assert_array_equal(to_host(res.perm.sorted_pair), sp)
    ex = oracle.Experts(inp["Wgate"], inp["Wup"], inp["Wdown"])
    ref = oracle.moe_forward(inp["x"], ex, ids_ref, w_ref, tokens=tokens)
    got = out_to_f64(res.out)
    if tokens is not None:
        got = got[np.asarray(tokens)]
    assert np.all(np.isfinite(got))
    assert_close_rel_max(got, ref, rel, spec.name)
    return counts


def test_f32_layer_odd_sizes():
    # d and f not multiples of 8 or of the tiles: the fp32 GEMMs' edge guards and the general
    # (4-element) combine path
    spec = synth.TINY_F32.with_(name="f32_T50_d100_f60_E4_k2", T=50, d=100, f=60, E=4)
    inp = layer_inputs(spec)
    for layout in ("slots", "permuted", "acc_f32"):
        log(spec.name, layout)
        res = _run_gpu(spec, inp, layout)
        _check_layer(spec, inp, res, 1e-4)


def test_tiny_f32_layer():
    spec = synth.TINY_F32
    inp = layer_inputs(spec)
    for layout in ("slots", "permuted", "acc_f32"):
        log("tiny f32", layout)
        res = _run_gpu(spec, inp, layout)
        _check_layer(spec, inp, res, 1e-4)


SMALL_BF16 = [
    synth.TINY_F32.with_(name="bf16_T300_d256_f384_E8_k2", dtype="bf16", T=300, d=256, f=384),
    synth.SKEWED_128E.with_(name="bf16_skew_T1000_d512_f256_E16_k4", T=1000, d=512, f=256, E=16,
                            k=4),
    synth.TINY_F32.with_(name="bf16_T2000_d384_f640_E4_k1", dtype="bf16", T=2000, d=384, f=640,
                         E=4, k=1),
    synth.TINY_F32.with_(name="bf16_T5_d128_f128_E8_k2", dtype="bf16", T=5, d=128, f=128),
    synth.MIXTRAL_PREFILL.with_(name="bf16_router_T600_d512_f1024_E8_k2", T=600, d=512, f=1024),
    # degenerate topologies: one expert (a dense gated MLP, routing weight 1) and every token on
    # every expert (k = E), each on the tiled GEMMs (P > 256) and the small-batch kernels
    synth.TINY_F32.with_(name="bf16_dense_T300_d256_f384_E1_k1", dtype="bf16", T=300, d=256,
                         f=384, E=1, k=1),
    synth.TINY_F32.with_(name="bf16_dense_T20_d256_f256_E1_k1", dtype="bf16", T=20, d=256, f=256,
                         E=1, k=1),
    synth.TINY_F32.with_(name="bf16_all_T100_d256_f256_E4_k4", dtype="bf16", T=100, d=256, f=256,
                         E=4, k=4),
    synth.TINY_F32.with_(name="bf16_all_T16_d256_f256_E4_k4", dtype="bf16", T=16, d=256, f=256,
                         E=4, k=4),
    # a single token: one row per selected expert, every other expert empty
    synth.TINY_F32.with_(name="bf16_one_T1_d256_f256_E8_k2", dtype="bf16", T=1, d=256, f=256,
                         E=8, k=2),
]


@pytest.mark.parametrize("spec", SMALL_BF16, ids=lambda s: s.name)
def test_small_bf16_layers(spec):
    inp = layer_inputs(spec)
    for layout in ("slots", "permuted", "acc_f32"):
        log(spec.name, layout)
        res = _run_gpu(spec, inp, layout)
        _check_layer(spec, inp, res, 2e-2)


# Shapes whose last round of tiles is cut along K (few tiles per XCD, long K): gate/up cut 8 ways,
# down cut 8 ways, and both GEMMs cut (2 and 4 ways). The cut tiles are summed in piece order by
# whichever piece finishes last, so repeated runs must agree bit for bit.
CUT_TAIL = [
    synth.TINY_F32.with_(name="bf16_cut_gateup_T200_d4096_f512_E2_k2", dtype="bf16", T=200,
                         d=4096, f=512, E=2, k=2),
    synth.TINY_F32.with_(name="bf16_cut_down_T200_d512_f4096_E2_k2", dtype="bf16", T=200, d=512,
                         f=4096, E=2, k=2),
    synth.TINY_F32.with_(name="bf16_cut_both_T700_d1024_f2048_E4_k2", dtype="bf16", T=700,
                         d=1024, f=2048, E=4, k=2),
]


@pytest.mark.parametrize("spec", CUT_TAIL, ids=lambda s: s.name)
def test_cut_tail_tiles(spec):
    inp = layer_inputs(spec)
    first = None
    for layout in ("slots", "acc_f32", "slots"):
        log(spec.name, layout)
        res = _run_gpu(spec, inp, layout)
        _check_layer(spec, inp, res, 2e-2)
        if layout == "slots":
            out = to_host(res.out)
            if first is None:
                first = out
            else:
                np.testing.assert_array_equal(out, first)


def test_bf16_prefill_kernel_on_small_batch_shapes():
    # P <= 256 goes to the decode kernels; d not a multiple of 128 forces the tiled kernels.
    spec = synth.TINY_F32.with_(name="bf16_T40_d192_f320_E8_k2", dtype="bf16", T=40, d=192,
                                f=320)
    inp = layer_inputs(spec)
    res = _run_gpu(spec, inp)
    _check_layer(spec, inp, res, 2e-2)


def test_decode_kernel_many_tokens_per_expert():
    # all 128 tokens on 2 experts -> token passes of 64 in the decode kernels
    spec = synth.TINY_F32.with_(name="bf16_decode_T128_d256_f512_E4_k2", dtype="bf16", T=128,
                                d=256, f=512, E=4, k=2, skew=6.0)
    inp = layer_inputs(spec)
    res = _run_gpu(spec, inp)
    counts = _check_layer(spec, inp, res, 2e-2)
    assert counts.max() > 64


@pytest.mark.parametrize("E", [16, 8])
def test_decode_skewed_partial_token_groups(E):
    # 128 pairs, skewed: two experts hold 50-64 tokens (a pass of 64 with its last group of 16
    # partly filled), the rest a few each (streaming gate/up kernel), the others none.
    spec = synth.TINY_F32.with_(name="bf16_decode_skew_T64_d256_f512_E%d_k2" % E, dtype="bf16",
                                T=64, d=256, f=512, E=E, k=2, skew=3.0)
    inp = layer_inputs(spec)
    ids, _ = oracle.route(inp["logits"], spec.k)
    counts = np.bincount(ids.reshape(-1), minlength=spec.E)
    assert counts.max() > 48 and ((counts > 0) & (counts <= 16)).any() and (counts == 0).any(), \
        counts
    for layout in ("slots", "acc_f32"):
        log(spec.name, layout, counts.tolist())
        res = _run_gpu(spec, inp, layout)
        _check_layer(spec, inp, res, 2e-2)


def test_decode_mixed_small_and_large_experts():
    # Skewed routing at a decode-sized batch: some experts get at most 16 tokens (streaming
    # kernel), others more (the multi-pass kernel); both run in one call, K a multiple of 256.
    spec = synth.SKEWED_128E.with_(name="bf16_decode_mixed_T100_d512_f1024_E8_k2", T=100, d=512,
                                   f=1024, E=8, k=2)
    inp = layer_inputs(spec)
    ids, _ = oracle.route(inp["logits"], spec.k)
    counts = np.bincount(ids.reshape(-1), minlength=spec.E)
    assert counts.max() > 16 and ((counts > 0) & (counts <= 16)).any(), counts
    for layout in ("slots", "permuted", "acc_f32"):
        log(spec.name, layout, counts.tolist())
        res = _run_gpu(spec, inp, layout)
        _check_layer(spec, inp, res, 2e-2)


def test_mixtral_decode_full():
    spec = synth.MIXTRAL_DECODE
    log("generating", spec.name)
    inp = layer_inputs(spec)
    for layout in ("slots", "permuted"):
        res = _run_gpu(spec, inp, layout)
        _check_layer(spec, inp, res, 2e-2)


def test_mixtral_prefill_full_sampled():
    spec = synth.MIXTRAL_PREFILL
    log("generating", spec.name)
    inp = layer_inputs(spec)
    res = _run_gpu(spec, inp)
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(spec.T, 24, replace=False)).tolist() + [0, spec.T - 1]
    _check_layer(spec, inp, res, 2e-2, tokens=tokens)
    # every output row is finite and not all zero
    out = out_to_f64(res.out)
    assert np.all(np.isfinite(out)) and np.all(np.abs(out).max(1) > 0)


def test_skewed_layer_reduced_full_compare_and_determinism():
    spec = synth.SKEWED_128E.with_(name="skewed_T2048_d512_f256_E128_k8", T=2048, d=512, f=256)
    inp = layer_inputs(spec)
    res = _run_gpu(spec, inp)
    counts = _check_layer(spec, inp, res, 2e-2)
    assert (counts == 0).sum() > 0
    res2 = _run_gpu(spec, inp)
    assert torch.equal(res.out, res2.out)  # slots layout: bit-identical reruns


def test_skewed_full_sampled():
    spec = synth.SKEWED_128E
    log("generating", spec.name)
    inp = layer_inputs(spec)
    res = _run_gpu(spec, inp)
    rng = np.random.default_rng(1)
    tokens = np.sort(rng.choice(spec.T, 64, replace=False))
    counts = _check_layer(spec, inp, res, 2e-2, tokens=tokens)
    log("skewed counts: max %d, empty %d" % (counts.max(), (counts == 0).sum()))
