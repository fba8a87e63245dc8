"""GPU parity of the fine-grained FP8 layer against the oracle.

Weights: fp32 masters from the generator, quantised to e4m3 with 128x128 block scales on the GPU
(fp8_quantize_weight) and, independently, by the oracle; the codes and scales must agree
bit-exactly, and the oracle then uses its own quantised weights. Activations: x is quantised per
token per 128 channels by fp8_quantize_act inside the layer; the oracle applies the same rule to x
and to h. Output bound: max|err| <= 6e-2 * max|ref| (the oracle of the quantised rule).
Every test runs with fp32 block scales and with UE8M0 scales (e8m0 bytes, powers of two; the
Transformers "Fine-grained FP8" page, section "UE8M0 scale format"), which the matrix unit applies
itself.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_softmax_amd as moe
import oracle
import synth
from gpu_util import (assert_close_rel_max, check_edge_rows_permuted, log, out_to_f64, to_dev,
                      to_host)

pytestmark = pytest.mark.gpu


FMTS = ("f32", "ue8m0")


def _quantise_on_gpu(masters, fmt="f32"):
    q, s = moe.fp8_quantize_weight(to_dev(masters), scale_fmt=fmt)
    return q, s


def _run_layer(x, logits, wq, k, y_layout="slots"):
    (qg, sg), (qu, su), (qd, sd) = wq
    res = moe.moe_layer(to_dev(x), qg, qu, qd, k, logits=to_dev(logits), s_gate=sg, s_up=su,
                        s_down=sd, y_layout=y_layout)
    torch.cuda.synchronize()
    return res


SMALL = [
    synth.DSV3_FP8.with_(name="fp8_T300_d512_f256_E16_k4", T=300, d=512, f=256, E=16, k=4),
    synth.DSV3_FP8.with_(name="fp8_T1000_d384_f640_E8_k2", T=1000, d=384, f=640, E=8, k=2),
    synth.DSV3_FP8.with_(name="fp8_T7_d256_f128_E4_k1", T=7, d=256, f=128, E=4, k=1),
    # one expert (small-batch kernels) and k = E (tiled GEMMs)
    synth.DSV3_FP8.with_(name="fp8_dense_T16_d256_f128_E1_k1", T=16, d=256, f=128, E=1, k=1),
    synth.DSV3_FP8.with_(name="fp8_all_T100_d256_f128_E4_k4", T=100, d=256, f=128, E=4, k=4),
    synth.DSV3_FP8.with_(name="fp8_one_T1_d256_f128_E8_k2", T=1, d=256, f=128, E=8, k=2),
    # skewed loads: experts of 531, 403, 289, 206, 168, 158, 134, 111 rows. With UE8M0 scales
    # (256-row tiles) two 256-row tiles and a 19-row remainder tile, a 256-row tile of 147 rows, a
    # 256-row tile plus a 33-row remainder, 256-row tiles whose last wave rows hold no rows, one
    # 128-row tile; with fp32 scales 128-row tiles with ragged tails. K = 384 and 640 take an odd
    # number of stages, N = 384 a down tile half past the weights
    synth.DSV3_FP8.with_(name="fp8_skew_T1000_d384_f640_E8_k2", T=1000, d=384, f=640, E=8, k=2,
                         skew=0.6),
    # experts of 569, 465, 353, 254, 223, 213, 170, 153 rows; even stage counts
    synth.DSV3_FP8.with_(name="fp8_skew_T1200_d512_f256_E8_k2", T=1200, d=512, f=256, E=8, k=2,
                         skew=0.5),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_small_fp8_layers(spec, fmt):
    log(spec.name, fmt)
    x = synth.gen_x(spec)
    logits = synth.gen_logits(spec)
    masters = [synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down")]
    wq = [_quantise_on_gpu(m, fmt) for m in masters]
    wq_ref = [oracle.quantize_weight(m, scale_fmt=fmt) for m in masters]
    for (q, s), (qr, sr) in zip(wq, wq_ref):
        np.testing.assert_array_equal(to_host(s), sr)
        np.testing.assert_array_equal(to_host(q), qr)
    ids_ref, w_ref = oracle.route(logits, spec.k)
    ex = oracle.Experts(*(q for q, _ in wq_ref), *(s for _, s in wq_ref), quant_act=True,
                        scale_fmt=fmt)
    ref = oracle.moe_forward(x, ex, ids_ref, w_ref)
    for layout in ("slots", "permuted", "acc_f32"):
        res = _run_layer(x, logits, wq, spec.k, layout)
        np.testing.assert_array_equal(to_host(res.topk_ids), ids_ref)
        got = out_to_f64(res.out)
        assert np.all(np.isfinite(got))
        assert_close_rel_max(got, ref, 6e-2, "%s %s %s" % (spec.name, fmt, layout))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xdt", ("bf16", "f32"))
def test_quantize_act_bit_exact(fmt, xdt):
    # codes and scales of the activation rule, with and without the row gather, against the
    # oracle's quantiser on the same inputs (bit for bit)
    spec = synth.DSV3_FP8.with_(T=333, d=640)
    x = synth.gen_x(spec)
    if xdt == "f32":
        x = synth.bf16_bits_to_f32(x) * np.float32(37.5)
    rows = np.random.default_rng(9).integers(0, spec.T, 500).astype(np.int32)
    log("quantize_act", fmt, xdt)
    for idx in (None, rows):
        q, s = moe.fp8_quantize_act(to_dev(x), row_index=None if idx is None else to_dev(idx),
                                    scale_fmt=fmt)
        torch.cuda.synchronize()
        xr = x if idx is None else x[idx]
        qr, sr = oracle.quantize_act(xr, scale_fmt=fmt)
        np.testing.assert_array_equal(to_host(s), sr)
        np.testing.assert_array_equal(to_host(q), qr)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_hidden_codes_match_oracle_rule(fmt):
    # The gate/up GEMM's h codes/scales, dequantised, stay within one e4m3 rounding step of the
    # oracle's h (computed in fp64 before quantisation) for every pair.
    spec = SMALL[0]
    x = synth.gen_x(spec)
    logits = synth.gen_logits(spec)
    masters = [synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down")]
    wq = [_quantise_on_gpu(m, fmt) for m in masters]
    (qg, sg), (qu, su), (qd, sd) = wq
    ids, w, _ = moe.moe_route(spec.k, logits=to_dev(logits))
    perm = moe.moe_permute(ids, spec.E)
    xq, xs = moe.fp8_quantize_act(to_dev(x), scale_fmt=fmt)
    ws = torch.empty(moe.experts_workspace_bytes(spec.T, spec.d, spec.f, spec.E, spec.k,
                                                 moe.MOE_FP8_E4M3, moe.MOE_FP8_E4M3),
                     dtype=torch.uint8, device="cuda")
    moe.moe_experts_forward(xq, qg, qu, qd, perm.offsets, perm.sorted_pair, w, spec.k,
                            x_scales=xs, s_gate=sg, s_up=su, s_down=sd, workspace=ws,
                            scale_fmt=fmt)
    torch.cuda.synchronize()
    P, f = spec.P, spec.f
    # workspace layout: two 256-byte-aligned tile tables, then h codes [P, f], then h scales
    off_h = 2 * ((spec.E + 1) * 4 + 255) // 256 * 256
    hq = to_host(ws[off_h:off_h + P * f]).reshape(P, f)
    off_s = off_h + (P * f + 255) // 256 * 256
    # (fp32 scale values in both formats; with UE8M0 they are powers of two)
    hs = to_host(ws[off_s:off_s + P * (f // 128) * 4].view(torch.float32)).reshape(P, f // 128)
    if fmt == "ue8m0":
        assert np.all(np.frexp(hs)[0] == 0.5)
    h_gpu = oracle.e4m3_decode_array(hq) * np.repeat(hs.astype(np.float64), 128, axis=1)
    sp = to_host(perm.sorted_pair)
    wr = [oracle.quantize_weight(m, scale_fmt=fmt) for m in masters]
    ex = oracle.Experts(*(q for q, _ in wr), *(s for _, s in wr), quant_act=True, scale_fmt=fmt)
    ids_h = to_host(ids).reshape(-1)
    h_ref, _ = oracle.expert_pairs(x, ex, sp // spec.k, ids_h[sp], want_y=False)
    # one e4m3 step is 2^-3 relative (normal range) plus the group scale's subnormal step
    bound = np.abs(h_ref) * 2.0 ** -3 + np.repeat(hs.astype(np.float64), 128, axis=1) * 2.0 ** -8
    assert np.all(np.abs(h_gpu - h_ref) <= bound + 1e-3 * np.abs(h_ref).max())


@pytest.mark.parametrize("fmt", FMTS)
def test_dsv3_fp8_full_sampled(fmt):
    spec = synth.DSV3_FP8
    T, d, f, E, k = spec.T, spec.d, spec.f, spec.E, spec.k
    log("generating", spec.name)
    x = synth.gen_x(spec)
    logits = synth.gen_logits(spec)
    ids_ref, w_ref = oracle.route(logits, k)
    rng = np.random.default_rng(2)
    tokens = np.sort(rng.choice(T, 12, replace=False))
    cnt = np.bincount(ids_ref.reshape(-1), minlength=E)
    need = sorted(set(ids_ref[tokens].reshape(-1).tolist()) | {int(cnt.argmax()), int(cnt.argmin())})
    remap = {e: i for i, e in enumerate(need)}
    # quantise expert by expert on the GPU; keep the oracle's own quantisation of the experts the
    # sampled tokens use, and check those bit-exactly against the GPU's
    dev_q, dev_s, ref_q, ref_s = {}, {}, {}, {}
    for which in ("gate", "up", "down"):
        rows, cols = (f, d) if which != "down" else (d, f)
        qt = torch.empty((E, rows, cols), dtype=torch.uint8, device="cuda")
        sdt = (torch.uint8, np.uint8) if fmt == "ue8m0" else (torch.float32, np.float32)
        st = torch.empty((E, rows // 128, cols // 128), dtype=sdt[0], device="cuda")
        rq = np.empty((len(need), rows, cols), np.uint8)
        rs = np.empty((len(need), rows // 128, cols // 128), sdt[1])
        for e0 in range(0, E, 16):
            chunk = list(range(e0, e0 + 16))
            m = synth.gen_expert_weight(spec, which, experts=chunk)
            q, s = moe.fp8_quantize_weight(to_dev(m), scale_fmt=fmt)
            qt[e0:e0 + 16] = q
            st[e0:e0 + 16] = s
            sel = [e for e in chunk if e in remap]
            if sel:
                oq, os_ = oracle.quantize_weight(m[[e - e0 for e in sel]], scale_fmt=fmt)
                for i, e in enumerate(sel):
                    rq[remap[e]] = oq[i]
                    rs[remap[e]] = os_[i]
                np.testing.assert_array_equal(to_host(q[[e - e0 for e in sel]]), oq)
                np.testing.assert_array_equal(to_host(s[[e - e0 for e in sel]]), os_)
        dev_q[which], dev_s[which] = qt, st
        ref_q[which], ref_s[which] = rq, rs
    log("weights quantised; running the layer")
    res = moe.moe_layer(to_dev(x), dev_q["gate"], dev_q["up"], dev_q["down"], k,
                        logits=to_dev(logits), s_gate=dev_s["gate"], s_up=dev_s["up"],
                        s_down=dev_s["down"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(res.topk_ids), ids_ref)
    got = out_to_f64(res.out)[tokens]
    ex = oracle.Experts(ref_q["gate"], ref_q["up"], ref_q["down"], ref_s["gate"], ref_s["up"],
                        ref_s["down"], quant_act=True, scale_fmt=fmt)
    ids_sub = np.vectorize(remap.get)(ids_ref[tokens]).astype(np.int32)
    ref = oracle.moe_forward(x[tokens], ex, ids_sub, w_ref[tokens])
    assert_close_rel_max(got, ref, 6e-2, "%s %s" % (spec.name, fmt))
    # the edge rows of the 256-row tiles (and of their 128-row halves) of every expert the oracle
    # holds, per pair
    n = check_edge_rows_permuted(spec, x, logits, [dev_q[w] for w in ("gate", "up", "down")],
                                 [dev_s[w] for w in ("gate", "up", "down")], ex, remap, (128, 256),
                                 6e-2, "%s %s" % (spec.name, fmt), scale_fmt=fmt)
    assert n >= 4 * len(need)


# ---- small batches: the weight-streaming fp8 kernels (at most 16 rows per expert) -----------

DECODE = [
    synth.DSV3_FP8.with_(name="fp8dec_T32_d512_f384_E8_k2", T=32, d=512, f=384, E=8, k=2),
    # 12.5 rows per expert on average, skewed: one expert holds 178 tokens (several 64-token
    # passes), one 20, two 1, the others none
    synth.DSV3_FP8.with_(name="fp8dec_T200_d256_f256_E16_k1_skew", T=200, d=256, f=256, E=16, k=1,
                         skew=3.0),
    # the last batch of the small-batch kernels: 16 rows per expert
    synth.DSV3_FP8.with_(name="fp8dec_T64_d256_f256_E8_k2_switch", T=64, d=256, f=256, E=8, k=2),
    # P = 256, the largest batch the streaming kernels take
    synth.DSV3_FP8.with_(name="fp8dec_T64_d384_f640_E16_k4", T=64, d=384, f=640, E=16, k=4),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("spec", DECODE, ids=lambda s: s.name)
def test_fp8_decode_layers(spec, fmt):
    assert moe.experts_small_batch(spec.T, spec.d, spec.f, spec.E, spec.k, moe.MOE_FP8_E4M3,
                                   moe.MOE_FP8_E4M3) == 1
    test_small_fp8_layers(spec, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_first_tiled_batch(fmt):
    # one pair past the small-batch limit (16 rows per expert): the tiled GEMMs
    spec = synth.DSV3_FP8.with_(name="fp8_T65_d256_f256_E8_k2_switch", T=65, d=256, f=256, E=8,
                                k=2)
    assert moe.experts_small_batch(spec.T, spec.d, spec.f, spec.E, spec.k, moe.MOE_FP8_E4M3,
                                   moe.MOE_FP8_E4M3) == 0
    test_small_fp8_layers(spec, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_mixtral_fp8_decode_full_sampled(fmt):
    # the Mixtral-shaped decode layer (T=32, d=4096, f=14336, E=8, k=2) with its weights
    # quantised to e4m3 on the GPU (codes and scales checked bit-exactly against the oracle's);
    # the oracle runs on 8 sampled tokens
    spec = synth.MIXTRAL_DECODE
    T, d, f, E, k = spec.T, spec.d, spec.f, spec.E, spec.k
    x = synth.gen_x(spec)
    lg = oracle.router_logits(x, synth.gen_router_weight(spec))
    ids_ref, w_ref = oracle.route(lg, k)
    dev_q, dev_s, ref_q, ref_s = {}, {}, {}, {}
    for which in ("gate", "up", "down"):
        rows, cols = (f, d) if which != "down" else (d, f)
        sdt = (torch.uint8, np.uint8) if fmt == "ue8m0" else (torch.float32, np.float32)
        qt = torch.empty((E, rows, cols), dtype=torch.uint8, device="cuda")
        st = torch.empty((E, rows // 128, cols // 128), dtype=sdt[0], device="cuda")
        rq = np.empty((E, rows, cols), np.uint8)
        rs = np.empty((E, rows // 128, cols // 128), sdt[1])
        for e in range(E):
            m = synth.bf16_bits_to_f32(synth.gen_expert_weight(spec, which, experts=[e]))
            q, s = moe.fp8_quantize_weight(to_dev(m), scale_fmt=fmt)
            oq, os_ = oracle.quantize_weight(m, scale_fmt=fmt)
            np.testing.assert_array_equal(to_host(q), oq)
            np.testing.assert_array_equal(to_host(s), os_)
            qt[e], st[e], rq[e], rs[e] = q[0], s[0], oq[0], os_[0]
        dev_q[which], dev_s[which] = qt, st
        ref_q[which], ref_s[which] = rq, rs
    log("weights quantised; running the decode layer", fmt)
    res = moe.moe_layer(to_dev(x), dev_q["gate"], dev_q["up"], dev_q["down"], k,
                        logits=to_dev(lg), s_gate=dev_s["gate"], s_up=dev_s["up"],
                        s_down=dev_s["down"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(res.topk_ids), ids_ref)
    tokens = np.arange(0, T, 4)
    ex = oracle.Experts(ref_q["gate"], ref_q["up"], ref_q["down"], ref_s["gate"], ref_s["up"],
                        ref_s["down"], quant_act=True, scale_fmt=fmt)
    ref = oracle.moe_forward(x[tokens], ex, ids_ref[tokens], w_ref[tokens])
    assert_close_rel_max(out_to_f64(res.out)[tokens], ref, 6e-2, "mixtral fp8 decode %s" % fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_act_edge_groups_bit_exact(fmt):
    # groups that stress the scale rule: all zero (with -0), amax exactly 448 * 2^e and one ulp
    # above, fp32 subnormals (the UE8M0 byte clamps at 0), values near the fp32 maximum, a single
    # non-zero element, alternating signs
    rng = np.random.default_rng(17)
    rows = []
    z = np.zeros(128, np.float32)
    z[::3] = -0.0
    rows.append(z)
    for e in (-20, 0, 7):
        b = np.full(128, np.float32(448.0 * 2.0 ** e) / 3, np.float32)
        b[5] = np.float32(448.0 * 2.0 ** e)
        rows.append(b)
        c = b.copy()
        c[5] = np.nextafter(np.float32(448.0 * 2.0 ** e), np.float32(np.inf))
        rows.append(c)
    rows.append((rng.standard_normal(128) * 1e-41).astype(np.float32))   # subnormal
    rows.append((rng.standard_normal(128) * 1e37).astype(np.float32))    # near the top
    one = np.zeros(128, np.float32)
    one[77] = np.float32(-3.25)
    rows.append(one)
    rows.append(np.where(np.arange(128) % 2 == 0, 1.0, -1.0).astype(np.float32) * 0.01)
    rows.append(rng.standard_normal(128).astype(np.float32))
    assert len(rows) % 2 == 0
    x = np.stack(rows).reshape(-1, 256)
    q, s = moe.fp8_quantize_act(to_dev(x), scale_fmt=fmt)
    torch.cuda.synchronize()
    qr, sr = oracle.quantize_act(x, scale_fmt=fmt)
    np.testing.assert_array_equal(to_host(s), sr)
    np.testing.assert_array_equal(to_host(q), qr)
