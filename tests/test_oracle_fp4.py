"""Pins for the oracle's FP4 (E2M1) expert weights with MX (UE8M0, 32-wide) block scales.

Transformers "Experts backends" page (notes on FP8 and FP4 quantised experts, packed as int8, with
float32 or UE8M0 scales) and "Fine-grained FP8" page (section "UE8M0 scale format"; FP4 experts
with UE8M0 weight scales). The pages fix neither the FP4 element format's details nor a block
size; the readings (OCP E2M1, element 2j in the low nibble of byte j, one UE8M0 scale per 32 input
channels, scale = smallest power of two 2^e with 6 * 2^e >= amax) are this project's. Checks: the
E2M1 value table of the OCP format, encode round trips and ties, a hand-packed example, exact
rational scale bounds, the rounding error bound and the layer against a numpy evaluation.
"""
from fractions import Fraction

import numpy as np

import oracle
import synth

# OCP FP4 E2M1: codes 0..7 = +0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 the same negated
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_value_table():
    for c in range(16):
        v = oracle.e2m1_value(c)
        ref = E2M1_TABLE[c & 7] * (-1 if c & 8 else 1)
        assert v == ref and np.signbit(v) == bool(c & 8), c


def test_e2m1_encode_round_trip_ties_and_saturation():
    for c in range(16):
        assert oracle.e2m1_encode(np.float32(oracle.e2m1_value(c))) == c
    # midpoints between neighbouring magnitudes go to the even code
    for c in range(7):
        lo, hi = E2M1_TABLE[c], E2M1_TABLE[c + 1]
        mid = np.float32((lo + hi) / 2)
        want = c if c % 2 == 0 else c + 1
        assert oracle.e2m1_encode(mid) == want
        assert oracle.e2m1_encode(-mid) == 8 | want
        # just off the midpoint: the nearer value
        assert oracle.e2m1_encode(np.nextafter(mid, np.float32(0))) == c
        assert oracle.e2m1_encode(np.nextafter(mid, np.float32(10))) == c + 1
    for v in (6.0, 6.5, 7.0, 1e30, float("inf")):
        assert oracle.e2m1_encode(np.float32(v)) == 7
        assert oracle.e2m1_encode(np.float32(-v)) == 15


def test_mxfp4_hand_packed_example():
    # one row of 32 with amax 6: scale 2^0 (byte 127); values on the grid pack pairwise, the
    # first of each pair in the low nibble: 0.5 (code 1) then 1.0 (code 2) -> byte 0x21, etc.
    row = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -6.0] + [0.0] * 24, np.float32)[None, :]
    q, s = oracle.quantize_weight_mxfp4(row)
    assert s.tolist() == [[127]]
    assert q[0, :4].tolist() == [0x21, 0x43, 0x65, 0xF7]
    assert np.all(q[0, 4:] == 0)
    # doubling every value moves the scale one step up and keeps the codes
    q2, s2 = oracle.quantize_weight_mxfp4(row * 2)
    assert s2.tolist() == [[128]] and np.array_equal(q2, q)


def test_mxfp4_scale_bounds_and_error():
    W = synth.normal_f32(6001, (64, 256), 1 / 16)
    W[3, 32:64] = 0.0                                     # an all-zero block
    W[5, :32] *= np.float32(1e-30)                        # a tiny block
    q, s = oracle.quantize_weight_mxfp4(W)
    assert q.shape == (64, 128) and s.shape == (64, 8)
    assert s[3, 1] == 127 and np.all(q[3, 16:32] == 0)
    for n in range(64):
        for kb in range(8):
            blk = W[n, kb * 32:(kb + 1) * 32]
            A = Fraction(float(np.abs(blk).max()))
            if A == 0:
                continue
            sc = Fraction(2) ** (int(s[n, kb]) - 127)
            assert 6 * sc >= A > 3 * sc, (n, kb)
    deq = oracle.e2m1_decode_packed(q) * np.repeat(oracle.e8m0_decode_array(s), 32, axis=1)
    sv = np.repeat(oracle.e8m0_decode_array(s), 32, axis=1)
    # one mantissa bit: relative error <= 1/4 from the scale up, absolute <= s/4 below it
    err = np.abs(deq - W)
    assert np.all(err <= np.maximum(np.abs(W) * 0.25, 0.25 * sv) * (1 + 1e-12))


def test_fp4_layer_vs_numpy():
    # experts with FP4 weights and e4m3 activations (UE8M0 scales throughout) against a numpy
    # evaluation: weights decoded by the pinned table and scales, x and h quantised by the pinned
    # UE8M0 activation rule, fp64 matmuls
    spec = synth.DSV3_FP8.with_(T=5, d=256, f=128, E=3, k=2)
    x = synth.gen_x(spec)
    Wg, Wu, Wd = (synth.gen_expert_weight(spec, n) for n in ("gate", "up", "down"))
    (qg, sg), (qu, su), (qd, sd) = (oracle.quantize_weight_mxfp4(a) for a in (Wg, Wu, Wd))
    ex = oracle.Experts(qg, qu, qd, sg, su, sd, quant_act=True, scale_fmt="ue8m0", w_fp4=True)
    ids, w = oracle.route(synth.gen_logits(spec), 2)
    out = oracle.moe_forward(x, ex, ids, w)

    def deq(q, s):
        return oracle.e2m1_decode_packed(q) * np.repeat(oracle.e8m0_decode_array(s), 32, axis=-1)

    def fq(v):
        qq, ss = oracle.quantize_act(v.astype(np.float32), scale_fmt="ue8m0")
        return oracle.e4m3_decode_array(qq) * oracle.e8m0_decode_array(ss).repeat(128, 1)

    G, U, D = deq(qg, sg), deq(qu, su), deq(qd, sd)
    xq = fq(synth.bf16_bits_to_f32(x))
    ref = np.zeros((spec.T, spec.d))
    for t in range(spec.T):
        for j in range(2):
            e = ids[t, j]
            g = G[e] @ xq[t]
            u = U[e] @ xq[t]
            h = fq((g / (1 + np.exp(-g)) * u)[None, :])[0]
            ref[t] += float(w[t, j]) * (D[e] @ h)
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-11 * np.abs(ref).max())
