"""GPU parity of the router, the expert grouping and the fp8 quantisers, against the oracle.

Routing ids, counts, offsets, sorted_pair, pair_pos, gathered rows and fp8 codes/scales must be
bit-exact. Routing weights: within 1 ulp (both sides evaluate them in fp64 and round once).
Router logits computed on the device: within 1e-5 * max(1, |l|) of the oracle's (fp32 sums on the
device, fp64 in the oracle); the selection replayed by the oracle on the device's own logits is
bit-exact, and against the oracle's own logits only near-tie tokens may route differently.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_softmax_amd as moe
import oracle
import synth
from gpu_util import (assert_weights_ulp, check_routing, layer_inputs, log, logit_bound, to_dev,
                      to_host)

pytestmark = pytest.mark.gpu

ROUTE_CASES = [
    ("tiny_E8_k2", synth.TINY_F32),
    ("skewed_E128_k8", synth.SKEWED_128E),
    ("dsv3_E256_k8", synth.DSV3_FP8),
    ("E8_k1", synth.TINY_F32.with_(k=1, T=333)),
    ("E5_k3", synth.TINY_F32.with_(E=5, k=3, T=77)),
    ("E1000_k32", synth.TINY_F32.with_(E=1000, k=32, T=129)),
    ("E1024_k1", synth.TINY_F32.with_(E=1024, k=1, T=50)),
]


@pytest.mark.parametrize("name,spec", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_given_logits(name, spec):
    log("route", name, spec.T, spec.E, spec.k)
    logits = synth.gen_logits(spec)
    ids_ref, w_ref = oracle.route(logits, spec.k)
    ids, w, _ = moe.moe_route(spec.k, logits=to_dev(logits))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(ids), ids_ref)
    assert_weights_ulp(to_host(w), w_ref, what=name)


def test_route_ties_and_equal_logits():
    # all-equal rows, pairwise ties, and rows with one ulp differences
    T, E = 64, 16
    lg = np.zeros((T, E), np.float32)
    lg[1] = np.arange(E) % 4
    lg[2] = np.float32(1.0)
    lg[2, 7] = np.nextafter(np.float32(1.0), np.float32(2.0))
    lg[3:] = np.round(synth.normal_f32(77, (T - 3, E)) * 2) / 2
    # signed zeros tie like equal values; negative values, subnormals of both signs
    lg[4] = np.where(np.arange(E) % 3 == 0, np.float32(-0.0), np.float32(0.0))
    lg[4, 9] = np.float32(-1e-30)
    lg[5] = -np.abs(synth.normal_f32(78, (E,)))
    lg[6] = np.float32(1e-45) * (np.arange(E) % 5 - 2)
    lg[7] = np.float32(-3.0)
    lg[7, 2] = lg[7, 11] = np.float32(-0.0)
    for k in (1, 2, 5, 16):
        ids_ref, w_ref = oracle.route(lg, k)
        ids, w, _ = moe.moe_route(k, logits=to_dev(lg))
        np.testing.assert_array_equal(to_host(ids), ids_ref)
        assert_weights_ulp(to_host(w), w_ref, what="ties k=%d" % k)


@pytest.mark.parametrize("T", [32, 4096, 37])
def test_route_router_gemm(T):
    spec = synth.MIXTRAL_PREFILL.with_(T=T)
    x = synth.gen_x(spec)
    Wr = synth.gen_router_weight(spec)
    log("router gemm T=%d" % T)
    ids, w, lg = moe.moe_route(2, x=to_dev(x), w_router=to_dev(Wr))
    torch.cuda.synchronize()
    inp = {"x": x, "Wr": Wr}
    check_routing(spec.with_(k=2), inp, to_host(ids), to_host(w), to_host(lg),
                  "router gemm T=%d" % T)


# The vector router path needs d % 8 == 0 (16-byte rows); other d take the general kernel.
ROUTER_SHAPES = [
    ("bf16_d100_scalar", "bf16", 37, 100, 8),
    ("f32_d256_vector", "f32", 41, 256, 8),
    ("f32_d60_scalar", "f32", 19, 60, 5),
    ("bf16_d512_E20_vector", "bf16", 70, 512, 20),      # one block per token (T < 256)
    ("bf16_d256_T300_E12_vector_groups", "bf16", 300, 256, 12),  # 8-token groups (T >= 256)
]


@pytest.mark.parametrize("name,xdt,T,d,E", ROUTER_SHAPES, ids=[c[0] for c in ROUTER_SHAPES])
def test_route_router_gemm_shapes(name, xdt, T, d, E):
    spec = synth.MIXTRAL_PREFILL.with_(T=T, d=d, E=E)
    x = synth.gen_x(spec)
    if xdt == "f32":
        x = synth.bf16_bits_to_f32(x)
    Wr = synth.gen_router_weight(spec)
    log("router gemm", name)
    ids, w, lg = moe.moe_route(2, x=to_dev(x), w_router=to_dev(Wr))
    torch.cuda.synchronize()
    check_routing(spec.with_(k=2), {"x": x, "Wr": Wr}, to_host(ids), to_host(w), to_host(lg),
                  "router gemm " + name)


PERMUTE_CASES = [
    ("tiny", 64, 2, 8, None),
    ("mixtral_prefill", 4096, 2, 8, None),
    ("mixtral_decode", 32, 2, 8, None),
    ("skewed_full", 16384, 8, 128, "skew"),
    ("dsv3_full", 8192, 8, 256, None),
    ("one_pair", 1, 1, 4, None),
    ("all_one_expert", 3000, 1, 64, "one"),
    ("max_E_k", 700, 32, 1024, None),
    ("ragged_chunk", 1025, 3, 7, None),
    # scan threads walking 11-12 and 29-30 chunks each (batched loads with partial batches)
    ("chunk_runs_11_12", 6000, 8, 256, None),
    ("chunk_runs_29_30", 7500, 8, 512, None),
    # one-workgroup path (P <= 1024): many experts per thread in its scan, and its exact limit
    ("small_many_experts", 30, 32, 1024, None),
    ("small_limit", 512, 2, 8, None),
]


@pytest.mark.parametrize("name,T,k,E,kind", PERMUTE_CASES, ids=[c[0] for c in PERMUTE_CASES])
def test_permute_bit_exact(name, T, k, E, kind):
    log("permute", name, T, k, E)
    if kind == "skew":
        lg = synth.skewed_logits(4001, T, E, 2.0)
    else:
        lg = synth.normal_f32(900 + E, (T, E))
    ids, _ = oracle.route(lg, k)
    if kind == "one":
        ids[:] = 17
    counts, offsets, sp, pp = oracle.permute(ids, E)
    perm = moe.moe_permute(to_dev(ids), E)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(perm.counts), counts)
    np.testing.assert_array_equal(to_host(perm.offsets), offsets)
    np.testing.assert_array_equal(to_host(perm.sorted_pair), sp)
    np.testing.assert_array_equal(to_host(perm.pair_pos), pp)
    # run twice: identical (deterministic scatter)
    perm2 = moe.moe_permute(to_dev(ids), E)
    assert torch.equal(perm.sorted_pair, perm2.sorted_pair)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
def test_permute_gather_rows(dtype):
    T, k, E, d = 777, 3, 16, 256
    ids, _ = oracle.route(synth.normal_f32(55, (T, E)), k)
    _, _, sp, _ = oracle.permute(ids, E)
    if dtype == "bf16":
        x = synth.normal_bf16(56, (T, d))
        xs = None
    elif dtype == "f32":
        x = synth.normal_f32(56, (T, d))
        xs = None
    else:
        x, xs = oracle.quantize_act(synth.normal_f32(56, (T, d)))
    perm = moe.moe_permute(to_dev(ids), E, x=to_dev(x), x_scales=None if xs is None else to_dev(xs))
    np.testing.assert_array_equal(to_host(perm.x_perm), x[sp // k])
    if xs is not None:
        np.testing.assert_array_equal(to_host(perm.x_perm_scales), xs[sp // k])


@pytest.mark.parametrize("T,k,E", [(100, 2, 8), (1500, 3, 16)], ids=["one_workgroup", "chunked"])
def test_permute_out_of_range_ids(T, k, E):
    """Ids outside [0, E) are contained: left out of the counts and the scatter, pair_pos -1,
    offsets[E] = number of in-range pairs, and the combine skips them."""
    log("permute_bad_ids", T, k, E)
    ids, w = oracle.route(synth.normal_f32(77, (T, E)), k)
    rng = np.random.default_rng(78)
    bad = rng.random(ids.shape) < 0.1
    ids[bad] = rng.choice(np.array([-1, E, E + 5, -(2 ** 31), 2 ** 31 - 1], np.int32), bad.sum())
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < E)
    nv = int(ok.sum())
    assert 0 < nv < flat.size
    d = 64
    x = synth.normal_bf16(79, (T, d))
    perm = moe.moe_permute(to_dev(ids), E, x=to_dev(x))
    torch.cuda.synchronize()
    counts = np.bincount(flat[ok], minlength=E).astype(np.int32)
    np.testing.assert_array_equal(to_host(perm.counts), counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    np.testing.assert_array_equal(to_host(perm.offsets), offsets)
    valid_pairs = np.nonzero(ok)[0]
    sp = valid_pairs[np.argsort(flat[valid_pairs], kind="stable")].astype(np.int32)
    np.testing.assert_array_equal(to_host(perm.sorted_pair)[:nv], sp)
    pp = np.full(flat.size, -1, np.int32)
    pp[sp] = np.arange(nv, dtype=np.int32)
    np.testing.assert_array_equal(to_host(perm.pair_pos), pp)
    np.testing.assert_array_equal(to_host(perm.x_perm)[:nv], x[sp // k])
    # combine over the permuted rows: the left-out pairs add nothing
    y = torch.zeros((flat.size, d), dtype=torch.float32, device="cuda")
    y[:nv] = torch.from_numpy(synth.bf16_bits_to_f32(x[sp // k])).cuda()
    out = moe.moe_combine(y, "permuted", T, k, d, pair_pos=perm.pair_pos, topk_w=to_dev(w),
                          out_dtype=torch.float32)
    wv = np.where(ok.reshape(T, k), w, 0.0).astype(np.float32)
    xf = synth.bf16_bits_to_f32(x).astype(np.float32)
    expect = np.zeros((T, d), np.float32)
    for j in range(k):
        expect = (wv[:, j:j + 1] * xf + expect).astype(np.float32)
    np.testing.assert_allclose(to_host(out), expect, rtol=1e-6, atol=1e-6)


def _edge_values():
    vals = [0.0, -0.0, 448.0, -448.0, 1e-30, -1e-30, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10,
            3 * 2.0 ** -10, 1.0625, 1.1875, 17.0, 18.0, 19.0, 240.0, 232.0, 0.015625]
    for c in range(0x7E):  # midpoints of neighbouring positive codes, scaled so that s = 1
        vals.append((oracle.e4m3_value(c) + oracle.e4m3_value(c + 1)) / 2)
    return np.array(vals, np.float32)


def test_quantize_act_bit_exact():
    M, K = 300, 7168
    x = synth.normal_bf16(5100, (M, K))
    # row 0: an amax of 448 (s = 1) followed by the edge values, so the codes of midpoints and
    # subnormals are exercised exactly
    ev = _edge_values()
    row = np.zeros(K, np.float32)
    row[0] = 448.0
    row[1:1 + ev.size] = ev
    x[0] = synth.f32_to_bf16(row)
    q, s = moe.fp8_quantize_act(to_dev(x))
    q_ref, s_ref = oracle.quantize_act(x)
    np.testing.assert_array_equal(to_host(s), s_ref)
    np.testing.assert_array_equal(to_host(q), q_ref)
    # f32 input with exact midpoints (not representable in bf16)
    xf = synth.normal_f32(5101, (64, 256))
    xf[0, :] = 0
    xf[0, 0] = 448.0
    xf[0, 1:1 + ev.size] = ev
    q, s = moe.fp8_quantize_act(to_dev(xf))
    q_ref, s_ref = oracle.quantize_act(xf)
    np.testing.assert_array_equal(to_host(s), s_ref)
    np.testing.assert_array_equal(to_host(q), q_ref)
    # an all-zero group
    z = np.zeros((4, 128), np.float32)
    q, s = moe.fp8_quantize_act(to_dev(z))
    assert np.all(to_host(s) == 1.0) and np.all(to_host(q) == 0)


def test_quantize_act_row_gather():
    x = synth.normal_bf16(5102, (50, 512))
    idx = np.array([7, 7, 0, 49, 13], np.int32)
    q, s = moe.fp8_quantize_act(to_dev(x), row_index=to_dev(idx))
    q_ref, s_ref = oracle.quantize_act(x[idx])
    np.testing.assert_array_equal(to_host(q), q_ref)
    np.testing.assert_array_equal(to_host(s), s_ref)


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantize_weight_bit_exact(src):
    W = synth.normal_f32(5200, (3, 256, 384), 1 / 16)
    if src == "bf16":
        Wb = synth.f32_to_bf16(W)
        W_in, W_ref = Wb, synth.bf16_bits_to_f32(Wb)
    else:
        W_in, W_ref = W, W
    q, s = moe.fp8_quantize_weight(to_dev(W_in))
    q_ref, s_ref = oracle.quantize_weight(W_ref)
    np.testing.assert_array_equal(to_host(s), s_ref)
    np.testing.assert_array_equal(to_host(q), q_ref)
