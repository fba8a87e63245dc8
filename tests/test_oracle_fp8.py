"""Pins for the oracle's number formats and fine-grained FP8 rule.

Transformers "Fine-grained FP8" page, intro bullets: weights quantised to 8 bits per 128x128
block; activations per token per 128-wide group of input channels, with dynamic scales. The
format (OCP E4M3FN), absmax scaling s = amax/448 and round-to-nearest-even are readings of what the
page leaves open. Checks: exhaustive decode against torch's float8_e4m3fn (a library codec), encode
against torch's fp32->e4m3fn cast inside the finite range, bf16 decode against torch's bfloat16,
closed forms for exactly representable inputs, and error bounds.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode_array(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_round_trip_and_midpoints():
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(v):
            continue
        assert oracle.e4m3_encode(np.float32(v)) == c
    # midpoints between neighbouring positive codes go to the even code
    for c in range(0, 0x7E):
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)  # exact in fp32
        assert float(mid) == (lo + hi) / 2
        assert oracle.e4m3_encode(mid) == (c if c % 2 == 0 else c + 1)
        assert oracle.e4m3_encode(-mid) == 0x80 | (c if c % 2 == 0 else c + 1)


def test_e4m3_encode_vs_torch_cast():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 100,
        rng.standard_normal(20000).astype(np.float32) * 0.01,
        rng.uniform(-448, 448, 20000).astype(np.float32),
        np.float32(2.0) ** rng.integers(-12, 9, 2000).astype(np.float32),
    ])
    v = np.clip(v, -448, 448).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(x) for x in v], np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_saturates():
    for v in (448.0, 449.0, 463.9, 464.0, 500.0, 1e30, float("inf")):
        assert oracle.e4m3_encode(np.float32(v)) == 0x7E
        assert oracle.e4m3_encode(np.float32(-v)) == 0xFE


def test_bf16_decode_all_codes_vs_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(c)) for c in codes[::97]])
    r = ref[::97]
    ok = ~np.isnan(r)
    np.testing.assert_array_equal(got[ok], r[ok])
    assert np.all(np.isnan(got[~ok]))


def test_quantize_act_closed_forms():
    # Group of 128 whose amax is 3.5: s = 3.5/448 = 2^-7 exactly, so v/s = 128 v is exact and
    # values on the e4m3 grid times 2^-7 are reproduced exactly.
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float64)
    rng = np.random.default_rng(3)
    vals = rng.choice(grid[grid <= 448], size=(4, 256)) * rng.choice([-1, 1], size=(4, 256))
    vals[:, 0] = 448.0
    vals[:, 128] = -448.0
    x = (vals * 2.0 ** -7).astype(np.float32)
    q, s = oracle.quantize_act(x)
    assert np.all(s == np.float32(3.5 / 448))
    np.testing.assert_array_equal(oracle.e4m3_decode_array(q) * s.repeat(128, 1), x)
    # an all-zero group gets scale 1 and zero codes
    z = np.zeros((2, 128), np.float32)
    qz, sz = oracle.quantize_act(z)
    assert np.all(sz == 1.0) and np.all(qz == 0)


def test_quantize_act_error_bound_and_bf16_input():
    x = synth.normal_bf16(5000, (64, 512))
    q, s = oracle.quantize_act(x)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    deq = oracle.e4m3_decode_array(q) * s.astype(np.float64).repeat(128, 1)
    amax = np.abs(xf).reshape(64, 4, 128).max(-1)
    np.testing.assert_array_equal(s, (amax / 448).astype(np.float32))
    # normal range: relative error <= 2^-4 (3 mantissa bits, round to nearest); subnormal range:
    # absolute error <= half a subnormal step times the scale
    err = np.abs(deq - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, 2.0 ** -10 * s.repeat(128, 1) * (1 + 1e-6))
    assert np.all(err <= bound * (1 + 1e-6))
    # the amax element of every group is exactly representable (it maps to 448)
    assert np.all((q.reshape(64, 4, 128) & 0x7F).max(-1) == 0x7E)


def test_quantize_weight_blocks():
    W = synth.normal_f32(5002, (256, 384), 1 / 16)
    q, s = oracle.quantize_weight(W)
    assert q.shape == (256, 384) and s.shape == (2, 3)
    for nb in range(2):
        for kb in range(3):
            blk = W[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert s[nb, kb] == np.float32(np.abs(blk).max() / np.float32(448))
            ref = torch.from_numpy(blk / s[nb, kb]).to(torch.float8_e4m3fn).view(torch.uint8)
            np.testing.assert_array_equal(
                q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128], ref.numpy())


def test_fp8_layer_lossless_special_case():
    """Inputs already on the e4m3 grid, with every weight block's and activation group's absmax
    equal to 448 * 2^m, quantise losslessly; the fp8 layer must then equal the unquantised layer
    on the same values (to double rounding). h is quantised too, so compare the first projection
    through the per-pair outputs and the layer with h-quantisation turned off."""
    rng = np.random.default_rng(11)
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float64)
    grid = grid[grid <= 448]
    T, d, f, E, k = 8, 256, 256, 4, 2

    def on_grid(shape, m, block_rows, block_cols):
        v = rng.choice(grid, size=shape) * rng.choice([-1, 1], size=shape) * 2.0 ** m
        # put the block maximum 448 * 2^m into every block
        for r0 in range(0, shape[-2], block_rows):
            for c0 in range(0, shape[-1], block_cols):
                v[..., r0, c0] = 448 * 2.0 ** m
        return v.astype(np.float32)

    x = on_grid((T, d), -7, 1, 128)
    Wg = on_grid((E, f, d), -10, 128, 128)
    Wu = on_grid((E, f, d), -10, 128, 128)
    Wd = on_grid((E, d, f), -10, 128, 128)
    qg, sg = oracle.quantize_weight(Wg)
    qu, su = oracle.quantize_weight(Wu)
    qd, sd = oracle.quantize_weight(Wd)
    ids, w = oracle.route(synth.normal_f32(5003, (T, E)), k)
    fp8 = oracle.Experts(qg, qu, qd, sg, su, sd, quant_act=False)
    ref = oracle.Experts(Wg, Wu, Wd)
    # weights and x are exactly representable -> identical to fp64 rounding
    np.testing.assert_allclose(oracle.moe_forward(x, fp8, ids, w),
                               oracle.moe_forward(x, ref, ids, w), rtol=1e-12, atol=1e-12)
    # the activation rule on x is lossless here as well
    qx, sx = oracle.quantize_act(x)
    np.testing.assert_array_equal(oracle.e4m3_decode_array(qx) * sx.repeat(128, 1), x)
    tok = np.repeat(np.arange(T), k).astype(np.int32)
    h_q, _ = oracle.expert_pairs(x, oracle.Experts(qg, qu, qd, sg, su, sd, quant_act=True), tok,
                                 ids.reshape(-1), want_y=False)
    h_r, _ = oracle.expert_pairs(x, ref, tok, ids.reshape(-1), want_y=False)
    np.testing.assert_allclose(h_q, h_r, rtol=1e-12, atol=1e-12)


def test_fp8_layer_quantises_h():
    # With quant_act the down projection sees h rounded by the 128-group rule: compare against the
    # unquantised layer evaluated on that rounded h (computed here from the per-pair outputs).
    spec = synth.DSV3_FP8.with_(T=6, d=256, f=256, E=4, k=2)
    x = synth.gen_x(spec)
    Wg, Wu, Wd = (synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down"))
    (qg, sg), (qu, su), (qd, sd) = (oracle.quantize_weight(a) for a in (Wg, Wu, Wd))
    ex = oracle.Experts(qg, qu, qd, sg, su, sd, quant_act=True)
    ids, w = oracle.route(synth.gen_logits(spec), 2)
    out = oracle.moe_forward(x, ex, ids, w)
    tok = np.repeat(np.arange(6), 2).astype(np.int32)
    h, _ = oracle.expert_pairs(x, ex, tok, ids.reshape(-1), want_y=False)
    hq, hs = oracle.quantize_act(h.astype(np.float32))
    hdq = oracle.e4m3_decode_array(hq) * hs.astype(np.float64).repeat(128, 1)
    Wd_deq = oracle.e4m3_decode_array(qd) * np.repeat(np.repeat(sd, 128, 1), 128, 2)
    y = np.einsum("pn,pon->po", hdq, Wd_deq[ids.reshape(-1)])
    ref = (y.reshape(6, 2, -1) * w[:, :, None].astype(np.float64)).sum(1)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


# ---- UE8M0 scale format ----------------------------------------------------------------------
# Transformers "Fine-grained FP8" page, section "UE8M0 scale format": block scales stored as
# float8_e8m0fnu bytes (powers of two). The choice of the power (the smallest 2^e with
# 448 * 2^e >= amax, for weight blocks and activation groups alike) is this project's reading.


def test_e8m0_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_decode_array(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_ue8m0_scale_is_smallest_covering_power_of_two():
    # exact rational check of 448 * s >= amax > 448 * s / 2, on random magnitudes, on the exact
    # boundaries 448 * 2^e and on their fp32 neighbours
    from fractions import Fraction
    rng = np.random.default_rng(21)
    amaxes = list(rng.lognormal(0.0, 8.0, 2000).astype(np.float32))
    for e in range(-30, 30):
        b = np.float32(448.0 * 2.0 ** e)
        amaxes += [b, np.nextafter(b, np.float32(np.inf)), np.nextafter(b, np.float32(0))]
    for a in amaxes:
        b = oracle.ue8m0_scale(np.float32(a))
        s = Fraction(2) ** (b - 127)
        A = Fraction(float(a))
        assert 448 * s >= A and 448 * s / 2 < A, (float(a), b)
    assert oracle.ue8m0_scale(np.float32(0.0)) == 127
    assert oracle.ue8m0_scale(np.float32(448.0)) == 127
    assert oracle.ue8m0_scale(np.float32(448.00003)) == 128
    assert oracle.ue8m0_scale(np.float32(224.0)) == 126


def test_quantize_act_ue8m0_closed_forms():
    # amax 448 * 2^-7: the scale is exactly 2^-7 (byte 120), codes equal the plain e4m3 encoding
    # of 128 v and values on the e4m3 grid times 2^-7 come back exactly.
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float64)
    rng = np.random.default_rng(23)
    vals = rng.choice(grid[grid <= 448], size=(4, 256)) * rng.choice([-1, 1], size=(4, 256))
    vals[:, 0] = 448.0
    vals[:, 128] = -448.0
    x = (vals * 2.0 ** -7).astype(np.float32)
    q, s = oracle.quantize_act(x, scale_fmt="ue8m0")
    assert s.dtype == np.uint8 and np.all(s == 120)
    np.testing.assert_array_equal(oracle.e4m3_decode_array(q) * 2.0 ** -7, x)
    # an amax just above 448 * 2^-7 moves to the next power: scale 2^-6, the amax maps to 224
    x2 = x.copy()
    x2[:, 0] = np.nextafter(np.float32(3.5), np.float32(4))
    q2, s2 = oracle.quantize_act(x2, scale_fmt="ue8m0")
    assert np.all(s2[:, 0] == 121) and np.all(s2[:, 1] == 120)
    assert np.all(oracle.e4m3_decode_array(q2[:, 0]) == 224.0)
    # an all-zero group: byte 127 (scale 1) and zero codes
    qz, sz = oracle.quantize_act(np.zeros((2, 128), np.float32), scale_fmt="ue8m0")
    assert np.all(sz == 127) and np.all(qz == 0)


def test_quantize_act_ue8m0_error_bound_and_torch_codes():
    x = synth.normal_bf16(5010, (64, 512))
    q, s = oracle.quantize_act(x, scale_fmt="ue8m0")
    xf = synth.bf16_bits_to_f32(x)
    sv = oracle.e8m0_decode_array(s).repeat(128, 1)
    # codes: torch's fp32 -> e4m3fn cast of the exactly scaled values (no value exceeds 448)
    scaled = (xf.astype(np.float64) / sv).astype(np.float32)
    assert np.abs(scaled).max() <= 448
    ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q, ref)
    # error: <= 2^-4 relative in the normal range, half a subnormal step times s below it
    deq = oracle.e4m3_decode_array(q) * sv
    err = np.abs(deq - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, 2.0 ** -10 * sv)
    assert np.all(err <= bound * (1 + 1e-6))
    # every group's scaled amax lies in (224, 448] (its code may round down to 224)
    smax = np.abs(scaled).reshape(64, 4, 128).max(-1)
    assert np.all((smax > 224) & (smax <= 448))
    top = np.abs(oracle.e4m3_decode_array(q).reshape(64, 4, 128)).max(-1)
    assert np.all((top >= 224) & (top <= 448))


def test_quantize_weight_ue8m0_blocks():
    W = synth.normal_f32(5011, (256, 384), 1 / 16)
    q, s = oracle.quantize_weight(W, scale_fmt="ue8m0")
    assert q.shape == (256, 384) and s.shape == (2, 3) and s.dtype == np.uint8
    from fractions import Fraction
    for nb in range(2):
        for kb in range(3):
            blk = W[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            A = Fraction(float(np.abs(blk).max()))
            sc = Fraction(2) ** (int(s[nb, kb]) - 127)
            assert 448 * sc >= A > 224 * sc
            scaled = (blk.astype(np.float64) / float(sc)).astype(np.float32)
            ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8)
            np.testing.assert_array_equal(
                q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128], ref.numpy())


def test_fp8_ue8m0_layer_vs_numpy():
    # The layer with UE8M0 scales against a numpy evaluation: scale bytes decoded as 2^(b-127)
    # (the pinned decode), x and h quantised by the pinned UE8M0 group rule, fp64 matmuls.
    spec = synth.DSV3_FP8.with_(T=6, d=256, f=256, E=4, k=2)
    x = synth.gen_x(spec)
    Wg, Wu, Wd = (synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down"))
    (qg, sg), (qu, su), (qd, sd) = (oracle.quantize_weight(a, scale_fmt="ue8m0")
                                    for a in (Wg, Wu, Wd))
    ex = oracle.Experts(qg, qu, qd, sg, su, sd, quant_act=True, scale_fmt="ue8m0")
    ids, w = oracle.route(synth.gen_logits(spec), 2)
    out = oracle.moe_forward(x, ex, ids, w)

    def deq_w(q, s):
        return oracle.e4m3_decode_array(q) * np.repeat(np.repeat(oracle.e8m0_decode_array(s), 128,
                                                                 -2), 128, -1)

    def fq(v):
        qq, ss = oracle.quantize_act(v.astype(np.float32), scale_fmt="ue8m0")
        return oracle.e4m3_decode_array(qq) * oracle.e8m0_decode_array(ss).repeat(128, 1)

    xq = fq(synth.bf16_bits_to_f32(x))
    G, U, D = deq_w(qg, sg), deq_w(qu, su), deq_w(qd, sd)
    ref = np.zeros((6, 256))
    for t in range(6):
        for j in range(2):
            e = ids[t, j]
            g = G[e] @ xq[t]
            u = U[e] @ xq[t]
            h = fq((g / (1 + np.exp(-g)) * u)[None, :])[0]
            ref[t] += float(w[t, j]) * (D[e] @ h)
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-11 * np.abs(ref).max())
