"""GPU parity of the whole layer (route -> permute -> grouped gated-MLP GEMMs -> combine) against
the oracle, through the C ABI.

Bounds (max over all compared output elements): bf16 layers max|err| <= 2e-2 * max|ref|;
the fp32 layer <= 1e-4 * max|ref| (fp32 end to end). Routing is checked against the oracle's own
routing (gpu_util.check_routing): ids bit-exact, weights within 1 ulp; where the router GEMM runs
on the device, its logits within 1e-5 * max(1, |l|) and only counted near-tie tokens may route
differently. Outputs are compared with the oracle evaluated on its own routing. Small shapes are
compared in full; the full-size workloads, in the launch configuration the benchmark times, on the
tokens that own the edge rows of the grouped GEMMs (every expert's first and last row, every row
tile's first and last row, every row of a small expert) plus a random sample.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_softmax_amd as moe
import oracle
import synth
from gpu_util import (assert_close_rel_max, check_routing, layer_inputs, log, out_to_f64,
                      targeted_tokens, to_dev, to_host)

pytestmark = pytest.mark.gpu


def _run_gpu(spec, inp, y_layout="slots"):
    dev = {k: to_dev(v) for k, v in inp.items()}
    res = moe.moe_layer(dev["x"], dev["Wgate"], dev["Wup"], dev["Wdown"], spec.k,
                        logits=dev.get("logits"), w_router=dev.get("Wr"), y_layout=y_layout)
    torch.cuda.synchronize()
    return res


def _check_layer(spec, inp, res, rel, tokens=None):
    """Routing, grouping and output of one layer run against the oracle. ``tokens``: compare the
    output on these tokens only (all tokens when None). Returns the oracle's expert counts."""
    ids_gpu = to_host(res.topk_ids)
    ids_ref, w_ref, keep = check_routing(
        spec, inp, ids_gpu, to_host(res.topk_w),
        None if "logits" in inp else to_host(res.logits), spec.name)
    # the grouping is a function of the device's ids (identical to the oracle's own where no
    # near tie flipped a token)
    counts, offsets, sp, pp = oracle.permute(ids_gpu, spec.E)
    np.testing.assert_array_equal(to_host(res.perm.counts), counts)
    np.testing.assert_array_equal(to_host(res.perm.offsets), offsets)
    np.testing.assert_array_equal(to_host(res.perm.sorted_pair), sp)
    np.testing.assert_array_equal(to_host(res.perm.pair_pos), pp)
    toks = np.arange(spec.T) if tokens is None else np.asarray(tokens)
    toks = toks[keep[toks]]
    ex = oracle.Experts(inp["Wgate"], inp["Wup"], inp["Wdown"])
    ref = oracle.moe_forward(inp["x"], ex, ids_ref, w_ref, tokens=toks)
    got = out_to_f64(res.out)[toks]
    assert np.all(np.isfinite(got))
    assert_close_rel_max(got, ref, rel, "%s (%d tokens)" % (spec.name, toks.size))
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
    # every expert (k = E), each on the tiled GEMMs and on the small-batch kernels (at most 12
    # rows per expert)
    synth.TINY_F32.with_(name="bf16_dense_T300_d256_f384_E1_k1", dtype="bf16", T=300, d=256,
                         f=384, E=1, k=1),
    synth.TINY_F32.with_(name="bf16_dense_T12_d256_f256_E1_k1", dtype="bf16", T=12, d=256, f=256,
                         E=1, k=1),
    synth.TINY_F32.with_(name="bf16_all_T100_d256_f256_E4_k4", dtype="bf16", T=100, d=256, f=256,
                         E=4, k=4),
    synth.TINY_F32.with_(name="bf16_all_T12_d256_f256_E4_k4", dtype="bf16", T=12, d=256, f=256,
                         E=4, k=4),
    # a single token: one row per selected expert, every other expert empty
    synth.TINY_F32.with_(name="bf16_one_T1_d256_f256_E8_k2", dtype="bf16", T=1, d=256, f=256,
                         E=8, k=2),
    # down projections with K = f >= 4096 run on four waves of 128x128: experts of ~120 rows
    # (the waves of the tile's second half hold no rows) and of 350 rows (a full and a ragged
    # row tile)
    synth.TINY_F32.with_(name="bf16_down4w_T300_d256_f8192_E5_k2", dtype="bf16", T=300, d=256,
                         f=8192, E=5, k=2),
    synth.TINY_F32.with_(name="bf16_down4w_T700_d256_f8192_E2_k1", dtype="bf16", T=700, d=256,
                         f=8192, E=2, k=1),
]


@pytest.mark.parametrize("spec", SMALL_BF16, ids=lambda s: s.name)
def test_small_bf16_layers(spec):
    inp = layer_inputs(spec)
    for layout in ("slots", "permuted", "acc_f32"):
        log(spec.name, layout)
        res = _run_gpu(spec, inp, layout)
        _check_layer(spec, inp, res, 2e-2)


# bf16 layers with fp32 expert outputs (y_dtype f32): the down epilogue's fp32 passes, on the
# eight-wave kernel and on the four-wave one (K = f >= 4096)
FP32_OUT = [
    synth.TINY_F32.with_(name="bf16_f32out_T300_d256_f1024_E5_k2", dtype="bf16", T=300, d=256,
                         f=1024, E=5, k=2),
    synth.TINY_F32.with_(name="bf16_f32out_T300_d256_f8192_E5_k2", dtype="bf16", T=300, d=256,
                         f=8192, E=5, k=2),
]


@pytest.mark.parametrize("spec", FP32_OUT, ids=lambda s: s.name)
def test_bf16_layers_fp32_outputs(spec):
    inp = layer_inputs(spec)
    dev = {k: to_dev(v) for k, v in inp.items()}
    for layout in ("slots", "permuted"):
        log(spec.name, layout, "fp32 y")
        res = moe.moe_layer(dev["x"], dev["Wgate"], dev["Wup"], dev["Wdown"], spec.k,
                            logits=dev.get("logits"), y_layout=layout, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert res.out.dtype == torch.float32
        _check_layer(spec, inp, res, 2e-2)


# Shapes whose last round of tiles is cut along K (few tiles per XCD, long K): gate/up cut 8 ways,
# down cut 8 ways, and both GEMMs cut (2 and 4 ways). A fix-up kernel sums each cut tile's pieces
# in piece order, so repeated runs must agree bit for bit.
CUT_TAIL = [
    synth.TINY_F32.with_(name="bf16_cut_gateup_T200_d4096_f512_E2_k2", dtype="bf16", T=200,
                         d=4096, f=512, E=2, k=2),
    synth.TINY_F32.with_(name="bf16_cut_down_T200_d512_f4096_E2_k2", dtype="bf16", T=200, d=512,
                         f=4096, E=2, k=2),
    synth.TINY_F32.with_(name="bf16_cut_both_T700_d1024_f2048_E4_k2", dtype="bf16", T=700,
                         d=1024, f=2048, E=4, k=2),
    synth.TINY_F32.with_(name="bf16_cut_down4w_T200_d512_f8192_E2_k2", dtype="bf16", T=200,
                         d=512, f=8192, E=2, k=2),
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
    # 10 rows per expert would take the small-batch kernels; d not a multiple of 128 forces the
    # tiled kernels.
    spec = synth.TINY_F32.with_(name="bf16_T40_d192_f320_E8_k2", dtype="bf16", T=40, d=192,
                                f=320)
    inp = layer_inputs(spec)
    res = _run_gpu(spec, inp)
    _check_layer(spec, inp, res, 2e-2)


def _assert_small_batch(spec, want=1):
    act = moe.MOE_F32 if spec.dtype == "f32" else moe.MOE_BF16
    assert moe.experts_small_batch(spec.T, spec.d, spec.f, spec.E, spec.k, act, act) == want, \
        spec.name


def test_decode_kernel_many_tokens_per_expert():
    # 8 rows per expert on average (small-batch kernels), skewed so that all 128 tokens sit on
    # two experts -> token passes of 64 in the decode kernels
    spec = synth.TINY_F32.with_(name="bf16_decode_T128_d256_f512_E32_k2", dtype="bf16", T=128,
                                d=256, f=512, E=32, k=2, skew=6.0)
    _assert_small_batch(spec)
    inp = layer_inputs(spec)
    res = _run_gpu(spec, inp)
    counts = _check_layer(spec, inp, res, 2e-2)
    assert counts.max() > 64


@pytest.mark.parametrize("E", [16, 12])
def test_decode_skewed_partial_token_groups(E):
    # 128 pairs, skewed: two experts hold 50-64 tokens (a pass of 64 with its last group of 16
    # partly filled), the rest a few each (streaming gate/up kernel), the others none.
    spec = synth.TINY_F32.with_(name="bf16_decode_skew_T64_d256_f512_E%d_k2" % E, dtype="bf16",
                                T=64, d=256, f=512, E=E, k=2, skew=3.0)
    _assert_small_batch(spec)
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
    spec = synth.SKEWED_128E.with_(name="bf16_decode_mixed_T100_d512_f1024_E24_k2", T=100, d=512,
                                   f=1024, E=24, k=2)
    _assert_small_batch(spec)
    inp = layer_inputs(spec)
    ids, _ = oracle.route(inp["logits"], spec.k)
    counts = np.bincount(ids.reshape(-1), minlength=spec.E)
    assert counts.max() > 16 and ((counts > 0) & (counts <= 16)).any(), counts
    for layout in ("slots", "permuted", "acc_f32"):
        log(spec.name, layout, counts.tolist())
        res = _run_gpu(spec, inp, layout)
        _check_layer(spec, inp, res, 2e-2)


def test_decode_streaming_limit_and_fp32_outputs():
    # Routing built so that expert 0 gets exactly 16 tokens (the most the streaming kernels take)
    # and expert 1 gets 17 (the K-split kernels), the others 5-6 each; bf16 and fp32 expert
    # outputs in every layout the down kernels store.
    spec = synth.TINY_F32.with_(name="bf16_decode_limit_T33_d256_f512_E8_k2", dtype="bf16", T=33,
                                d=256, f=512, E=8, k=2)
    _assert_small_batch(spec)
    inp = layer_inputs(spec)
    lg = np.random.default_rng(7).normal(0.0, 0.1, (spec.T, spec.E)).astype(np.float32)
    for t in range(spec.T):
        lg[t, 0 if t < 16 else 1] += 10.0
        lg[t, 2 + t % 6] += 9.0
    inp["logits"] = lg
    ids, _ = oracle.route(lg, spec.k)
    counts = np.bincount(ids.reshape(-1), minlength=spec.E)
    assert counts[0] == 16 and counts[1] == 17, counts
    for layout in ("slots", "permuted", "acc_f32"):
        log(spec.name, layout, counts.tolist())
        _check_layer(spec, inp, _run_gpu(spec, inp, layout), 2e-2)
    dev = {k: to_dev(v) for k, v in inp.items()}
    for layout in ("slots", "permuted"):
        log(spec.name, layout, "fp32 y")
        res = moe.moe_layer(dev["x"], dev["Wgate"], dev["Wup"], dev["Wdown"], spec.k,
                            logits=dev["logits"], y_layout=layout, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert res.out.dtype == torch.float32
        _check_layer(spec, inp, res, 2e-2)


def test_decode_two_token_passes():
    # At most 32 tokens: the streaming kernels take every expert (the K-split kernels are not
    # launched), expert 0 with 20 pairs in two passes (16 + 4), expert 1 with 12 in one.
    spec = synth.TINY_F32.with_(name="bf16_decode_passes_T32_d256_f512_E8_k2", dtype="bf16",
                                T=32, d=256, f=512, E=8, k=2)
    _assert_small_batch(spec)
    inp = layer_inputs(spec)
    lg = np.random.default_rng(11).normal(0.0, 0.1, (spec.T, spec.E)).astype(np.float32)
    for t in range(spec.T):
        lg[t, 0 if t < 20 else 1] += 10.0
        lg[t, 2 + t % 6] += 9.0
    inp["logits"] = lg
    ids, _ = oracle.route(lg, spec.k)
    counts = np.bincount(ids.reshape(-1), minlength=spec.E)
    assert counts[0] == 20 and counts[1] == 12, counts
    for layout in ("slots", "permuted", "acc_f32"):
        log(spec.name, layout, counts.tolist())
        _check_layer(spec, inp, _run_gpu(spec, inp, layout), 2e-2)


def test_decode_kernel_mix_when_d_is_not_a_stage_multiple():
    # d = 384 is a multiple of 128 but not of the gate/up streaming kernel's 256-wide stage: with
    # T <= 32 the gate/up projection runs on the K-split kernel for every expert while the down
    # projection streams every expert.
    spec = synth.TINY_F32.with_(name="bf16_decode_mix_T24_d384_f256_E4_k2", dtype="bf16", T=24,
                                d=384, f=256, E=4, k=2)
    _assert_small_batch(spec)
    inp = layer_inputs(spec)
    for layout in ("slots", "permuted", "acc_f32"):
        log(spec.name, layout)
        _check_layer(spec, inp, _run_gpu(spec, inp, layout), 2e-2)


def test_decode_repeated_expert_ids():
    # Routing ids that name one expert twice for a token (not what the router makes, but what the
    # permutation accepts): with 24 tokens expert 0 gets 44 pairs, three passes of the streaming
    # kernels; checked against the oracle's per-token sum over the given ids and weights.
    spec = synth.TINY_F32.with_(name="bf16_decode_repeat_T24_d256_f512_E4_k2", dtype="bf16",
                                T=24, d=256, f=512, E=4, k=2)
    _assert_small_batch(spec)
    inp = layer_inputs(spec)
    ids = np.zeros((spec.T, spec.k), dtype=np.int32)
    ids[20:, 1] = 1
    w = np.random.default_rng(5).uniform(0.2, 0.8, (spec.T, spec.k)).astype(np.float32)
    assert np.bincount(ids.reshape(-1), minlength=spec.E).tolist() == [44, 4, 0, 0]
    dev = {k: to_dev(v) for k, v in inp.items()}
    ids_d, w_d = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    perm = moe.moe_permute(ids_d, spec.E)
    ex = oracle.Experts(inp["Wgate"], inp["Wup"], inp["Wdown"])
    ref = oracle.moe_forward(inp["x"], ex, ids, w)
    for layout in ("slots", "permuted"):
        y = moe.moe_experts_forward(dev["x"], dev["Wgate"], dev["Wup"], dev["Wdown"], perm.offsets,
                                    perm.sorted_pair, w_d, spec.k, y_layout=layout)
        out = moe.moe_combine(y, layout, spec.T, spec.k, spec.d, pair_pos=perm.pair_pos,
                              topk_w=w_d, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert_close_rel_max(out_to_f64(out), ref, 2e-2, "%s %s" % (spec.name, layout))


@pytest.mark.parametrize("T,want", [(48, 1), (49, 0)])
def test_small_batch_switch_boundary(T, want):
    # the last batch of the small-batch kernels (12 rows per expert) and the first of the tiled
    # GEMMs, same layer otherwise
    spec = synth.MIXTRAL_DECODE.with_(name="bf16_switch_T%d_d512_f1024_E8_k2" % T, T=T, d=512,
                                      f=1024)
    _assert_small_batch(spec, want)
    inp = layer_inputs(spec)
    for layout in ("slots", "acc_f32"):
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
    tokens = targeted_tokens(to_host(res.perm.offsets), to_host(res.perm.sorted_pair), spec.k,
                             tile_rows=(256,), n_random=24, seed=0, T=spec.T)
    log("%s: comparing %d tokens" % (spec.name, tokens.size))
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
    offsets = to_host(res.perm.offsets)
    tokens = targeted_tokens(offsets, to_host(res.perm.sorted_pair), spec.k, tile_rows=(256,),
                             small=16, n_random=64, seed=1, T=spec.T)
    counts = np.diff(offsets)
    log("%s: comparing %d tokens; %d experts with 1-15 rows" % (
        spec.name, tokens.size, int(((counts > 0) & (counts < 16)).sum())))
    counts = _check_layer(spec, inp, res, 2e-2, tokens=tokens)
    log("skewed counts: max %d, empty %d" % (counts.max(), (counts == 0).sum()))
