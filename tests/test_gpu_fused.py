"""GPU checks of the fused small-batch path (moe_fused_forward: one routing kernel, no permutation).

The path computes what moe_route + moe_permute (+ fp8_quantize_act) + moe_experts_forward (slots)
+ moe_combine compute. Its routing ids and weights must be bit-identical to that sequence, and so
must its output wherever the sequence takes the same small-batch kernels (moe_experts_small_batch;
past that batch size the sequence takes the tiled GEMMs, whose rounding differs); each weight
format is also compared with the oracle here directly (bars as for the layer tests: 2e-2 * max|ref|
for bf16, 6e-2 for fp8 / FP4). Repeated calls on one workspace (filled with garbage first) check
that nothing depends on its previous contents.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_softmax_amd as moe
import oracle
import synth
from gpu_util import assert_close_rel_max, check_routing, log, out_to_f64, to_dev, to_host

pytestmark = pytest.mark.gpu


def _weights(spec, fmt):
    """Device weights (+ scales) in format fmt ('bf16', 'f32', 'ue8m0', 'fp4') and the oracle's
    expert set for them."""
    masters = [synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down")]
    if fmt == "bf16":
        dev = [to_dev(m) for m in masters]
        return dev, (None, None, None), oracle.Experts(*masters)
    f32 = [synth.bf16_bits_to_f32(m) if m.dtype == np.uint16 else m for m in masters]
    if fmt == "fp4":
        q = [moe.fp4_quantize_weight_mx(to_dev(m), tiled=True) for m in f32]
        qr = [oracle.quantize_weight_mxfp4(m) for m in f32]
        ex = oracle.Experts(*(a for a, _ in qr), *(b for _, b in qr), quant_act=True,
                            scale_fmt="ue8m0", w_fp4=True)
    else:
        q = [moe.fp8_quantize_weight(to_dev(m), scale_fmt=fmt) for m in f32]
        qr = [oracle.quantize_weight(m, scale_fmt=fmt) for m in f32]
        ex = oracle.Experts(*(a for a, _ in qr), *(b for _, b in qr), quant_act=True,
                            scale_fmt=fmt)
    return [a for a, _ in q], [b for _, b in q], ex


def _unfused(x, W, S, k, logits, wr, fmt, out_dtype):
    res = moe.moe_layer(x, *W, k, logits=logits, w_router=wr, s_gate=S[0], s_up=S[1],
                        s_down=S[2], out_dtype=out_dtype, w_fp4=fmt == "fp4")
    return res.out, res.topk_ids, res.topk_w


def _check_same(fused, unfused, what, out_too=True):
    """Bit-identical routing ids and weights, and output when out_too (the separate calls take the
    same small-batch kernels only while moe_experts_small_batch says so)."""
    for a, b, name in zip(fused, unfused, ("out", "topk_ids", "topk_w")):
        assert a.dtype == b.dtype and a.shape == b.shape, (what, name)
        if name == "out" and not out_too:
            continue
        assert torch.equal(a, b), "%s: fused %s differs from the unfused sequence" % (what, name)


def _separate_is_small_batch(spec, fmt):
    w = {"bf16": moe.MOE_BF16, "fp4": moe.MOE_FP4_E2M1}.get(fmt, moe.MOE_FP8_E4M3)
    act = moe.MOE_BF16 if fmt == "bf16" else moe.MOE_FP8_E4M3
    return moe.experts_small_batch(spec.T, spec.d, spec.f, spec.E, spec.k, act, w) == 1


CASES = [
    # bf16 weights: experts with <= 16 tokens (streaming gate/up kernel) and with more
    ("bf16", synth.MIXTRAL_DECODE.with_(name="fz_bf16_T24_d256_f512_E8_k2", T=24, d=256, f=512,
                                        E=8, k=2)),
    ("bf16", synth.MIXTRAL_DECODE.with_(name="fz_bf16_T100_d384_f256_E4_k2", T=100, d=384, f=256,
                                        E=4, k=2)),
    # skewed: experts of 44-64 tokens beside experts of a few and empty ones
    ("bf16", synth.MIXTRAL_DECODE.with_(name="fz_bf16_T64_d256_f512_E16_k2_skew", T=64, d=256,
                                        f=512, E=16, k=2, logits="given", skew=3.0)),
    ("bf16", synth.MIXTRAL_DECODE.with_(name="fz_bf16_T64_d256_f512_E8_k2_skew", T=64, d=256,
                                        f=512, E=8, k=2, logits="given", skew=2.0)),
    # at most 32 tokens: the streaming kernels take every expert, here 32 and 23 pairs in two
    # passes of 16 each, beside experts of 6, 2 and 1 and empty ones
    ("bf16", synth.MIXTRAL_DECODE.with_(name="fz_bf16_T32_d256_f512_E8_k2_skew", T=32, d=256,
                                        f=512, E=8, k=2, logits="given", skew=2.0)),
    ("f32", synth.DSV3_FP8.with_(name="fz_fp8_T32_d512_f384_E8_k2", T=32, d=512, f=384, E=8, k=2)),
    ("ue8m0", synth.DSV3_FP8.with_(name="fz_fp8ue_T32_d512_f384_E8_k2", T=32, d=512, f=384, E=8,
                                   k=2)),
    ("ue8m0", synth.DSV3_FP8.with_(name="fz_fp8ue_T64_d256_f640_E16_k4", T=64, d=256, f=640,
                                   E=16, k=4)),
    ("fp4", synth.DSV3_FP8.with_(name="fz_fp4_T32_d512_f384_E8_k2", T=32, d=512, f=384, E=8,
                                 k=2)),
    ("fp4", synth.DSV3_FP8.with_(name="fz_fp4_T1_d256_f128_E4_k1", T=1, d=256, f=128, E=4, k=1)),
    # many experts (several logits per lane in the top-k selection), P = 256
    ("fp4", synth.DSV3_FP8.with_(name="fz_fp4_T64_d256_f256_E64_k4", T=64, d=256, f=256, E=64,
                                 k=4)),
    ("ue8m0", synth.DSV3_FP8.with_(name="fz_fp8ue_T32_d512_f256_E256_k8_router", T=32, d=512,
                                   f=256, E=256, k=8, logits="router")),
]


@pytest.mark.parametrize("fmt,spec", CASES, ids=lambda c: c if isinstance(c, str) else c.name)
def test_fused_matches_unfused_and_oracle(fmt, spec):
    log(spec.name, fmt)
    x = to_dev(synth.gen_x(spec))
    W, S, ex = _weights(spec, fmt)
    if spec.logits == "router":
        wr_np = synth.gen_router_weight(spec)
        logits, wr = None, to_dev(wr_np)
        lg_np = oracle.router_logits(synth.gen_x(spec), wr_np)
    else:
        lg_np = synth.gen_logits(spec)
        logits, wr = to_dev(lg_np), None
    ref_seq = _unfused(x, W, S, spec.k, logits, wr, fmt, None)
    ws = None
    for call in range(3):   # one workspace, three calls
        lg_out = torch.empty((spec.T, spec.E), dtype=torch.float32, device="cuda") \
            if wr is not None else None
        n = moe.load_library().moe_fused_workspace_size(
            spec.T, spec.d, spec.f, spec.E, spec.k,
            {"bf16": moe.MOE_BF16, "fp4": moe.MOE_FP4_E2M1}.get(fmt, moe.MOE_FP8_E4M3),
            moe.MOE_BF16)
        if ws is None:
            ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")   # garbage contents
        got = moe.moe_fused_forward(x, *W, spec.k, logits=logits, w_router=wr, s_gate=S[0],
                                    s_up=S[1], s_down=S[2], w_fp4=fmt == "fp4", workspace=ws,
                                    logits_out=lg_out)
        torch.cuda.synchronize()
        _check_same(got, ref_seq, "%s %s call %d" % (spec.name, fmt, call),
                    _separate_is_small_batch(spec, fmt))
    # against the oracle's own routing (its own logits when the router GEMM ran on the device)
    inp = {"x": synth.gen_x(spec)}
    if wr is not None:
        inp["Wr"] = wr_np
    else:
        inp["logits"] = lg_np
    ids_ref, w_ref, keep = check_routing(spec, inp, to_host(got[1]), to_host(got[2]),
                                         to_host(lg_out) if wr is not None else None,
                                         "%s %s" % (spec.name, fmt))
    toks = np.flatnonzero(keep)
    ref = oracle.moe_forward(inp["x"], ex, ids_ref, w_ref, tokens=toks)
    assert_close_rel_max(out_to_f64(got[0])[toks], ref, 2e-2 if fmt == "bf16" else 6e-2,
                         "%s %s vs oracle" % (spec.name, fmt))


def test_fused_f32_output_and_max_pairs():
    # P = 256 (the largest batch), fp32 output, UE8M0 scales
    spec = synth.DSV3_FP8.with_(name="fz_T128_d256_f256_E8_k2", T=128, d=256, f=256, E=8, k=2)
    x = to_dev(synth.gen_x(spec))
    W, S, _ = _weights(spec, "ue8m0")
    logits = to_dev(synth.gen_logits(spec))
    ref_seq = _unfused(x, W, S, spec.k, logits, None, "ue8m0", torch.float32)
    got = moe.moe_fused_forward(x, *W, spec.k, logits=logits, s_gate=S[0], s_up=S[1],
                                s_down=S[2], out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_same(got, ref_seq, spec.name)


@pytest.mark.parametrize("fmt", ("f32", "ue8m0", "fp4"))
def test_fused_f32_activations(fmt):
    # fp32 x with fp8 / FP4 experts: quantised inside the routing kernel; fp32 output
    spec = synth.DSV3_FP8.with_(name="fz_xf32", T=20, d=384, f=256, E=8, k=2)
    x = to_dev(synth.bf16_bits_to_f32(synth.gen_x(spec)) * np.float32(1.5))
    W, S, _ = _weights(spec, fmt)
    logits = to_dev(synth.gen_logits(spec))
    ref_seq = _unfused(x, W, S, spec.k, logits, None, fmt, torch.float32)
    got = moe.moe_fused_forward(x, *W, spec.k, logits=logits, s_gate=S[0], s_up=S[1],
                                s_down=S[2], w_fp4=fmt == "fp4")
    torch.cuda.synchronize()
    assert got[0].dtype == torch.float32
    _check_same(got, ref_seq, "fp32 x " + fmt)


def test_fused_rejects_large_batches():
    spec = synth.DSV3_FP8.with_(name="fz_big", T=129, d=256, f=256, E=8, k=2)   # 258 pairs
    x = to_dev(synth.gen_x(spec))
    W, S, _ = _weights(spec.with_(T=4), "ue8m0")
    with pytest.raises(ValueError, match="UNSUPPORTED"):
        moe.moe_fused_forward(x, *W, spec.k, logits=to_dev(synth.gen_logits(spec)), s_gate=S[0],
                              s_up=S[1], s_down=S[2])


@pytest.mark.parametrize("fmt", ("bf16", "fp4"))
def test_mixtral_decode_fused_matches_unfused(fmt):
    # the Mixtral-shaped decode layer (router GEMM on the device) through both paths
    spec = synth.MIXTRAL_DECODE
    x = to_dev(synth.gen_x(spec))
    wr = to_dev(synth.gen_router_weight(spec))
    if fmt == "bf16":
        W, S = [to_dev(synth.gen_expert_weight(spec, n)) for n in ("gate", "up", "down")], \
            (None, None, None)
    else:
        W, S = [], []
        for n in ("gate", "up", "down"):
            q, s = moe.fp4_quantize_weight_mx(to_dev(synth.gen_expert_weight(spec, n)), tiled=True)
            W.append(q)
            S.append(s)
    ref_seq = _unfused(x, W, S, spec.k, None, wr, fmt, None)
    got = moe.moe_fused_forward(x, *W, spec.k, w_router=wr, s_gate=S[0], s_up=S[1], s_down=S[2],
                                w_fp4=fmt == "fp4")
    torch.cuda.synchronize()
    _check_same(got, ref_seq, "mixtral decode " + fmt)
