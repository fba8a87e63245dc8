"""Helpers for the GPU parity tests: host <-> device copies, cached workload inputs, the
tolerance check. Inputs come from ``synth``; expected values only from ``oracle``."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import synth

DEV = "cuda"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    a = to_host(t)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def assert_close_rel_max(got: np.ndarray, ref: np.ndarray, rel: float, what: str = ""):
    """max |got - ref| <= rel * max |ref| over all elements."""
    err = np.abs(got - ref).max()
    scale = np.abs(ref).max()
    log("%s max|err| = %.3e, max|ref| = %.3e, ratio = %.3e (bound %.1e)"
        % (what, err, scale, err / scale, rel))
    assert err <= rel * scale, (what, err, scale)


@functools.lru_cache(maxsize=4)
def layer_inputs(spec: synth.LayerSpec):
    """Host arrays for a workload (bf16 as uint16 bits, fp8 layers as fp32 masters)."""
    d = dict(x=synth.gen_x(spec))
    if spec.logits == "given":
        d["logits"] = synth.gen_logits(spec)
    else:
        d["Wr"] = synth.gen_router_weight(spec)
    for n in ("gate", "up", "down"):
        d["W" + n] = synth.gen_expert_weight(spec, n)
    return d


def oracle_experts(spec, inp):
    return oracle.Experts(inp["Wgate"], inp["Wup"], inp["Wdown"])


# ---- routing checks against the oracle ---------------------------------------------------------
#
# Router logits computed on the device (fp32 sums) may differ from the oracle's (fp64 sums, one
# rounding) by a few fp32 ulps of the partial sums; the bound below is 1e-5 relative for |l| >= 1
# with an absolute floor of 1e-5 (logits here are O(1): N(0, 1.28) for the Mixtral router).
LOGIT_REL = 1e-5


def logit_bound(lg_ref: np.ndarray) -> np.ndarray:
    return LOGIT_REL * np.maximum(1.0, np.abs(lg_ref.astype(np.float64)))


def assert_weights_ulp(got: np.ndarray, ref: np.ndarray, extra=None, what=""):
    """|got - ref| <= 1 ulp of ref (+ extra): the weights are computed in fp64 and rounded once
    on both sides, so they agree unless the exact value lies within ~1e-16 of a rounding
    boundary."""
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    ulp = np.spacing(np.abs(ref)).astype(np.float64)
    bound = ulp + (0.0 if extra is None else extra)
    diff = np.abs(got.astype(np.float64) - ref)
    n_exact = int((got == ref).sum())
    log("%s routing weights: %d of %d bit-identical, max |diff| / ulp = %.2f"
        % (what, n_exact, ref.size, float((diff / ulp).max()) if ref.size else 0.0))
    assert np.all(diff <= bound), (what, float((diff - bound).max()))


def check_routing(spec, inp, ids_gpu, w_gpu, lg_gpu=None, what=""):
    """Routing of a layer run against the oracle's own routing.

    Given logits: ids bit-exact, weights within 1 ulp. Logits computed on the device: the logits
    within logit_bound, the selection and weights replayed by the oracle on the device's logits
    exact (ids) / within 1 ulp (weights), and against the oracle's own logits the ids differ only
    for tokens whose oracle logits hold a near tie (adjacent top-(k+1) logits closer than twice the
    bound), which are counted and logged; on all other tokens the weights agree within the change
    that the logit difference can cause, |dw_j| <= 2 w_j max_i |dl_i| (+ 1 ulp).

    Returns (ids_ref, w_ref, keep): the oracle's own routing and a mask of the tokens whose ids
    match (all tokens when the logits are given).
    """
    k = spec.k
    ids_gpu = np.asarray(ids_gpu)
    w_gpu = np.asarray(w_gpu)
    if "logits" in inp:
        ids_ref, w_ref = oracle.route(inp["logits"], k)
        np.testing.assert_array_equal(ids_gpu, ids_ref)
        assert_weights_ulp(w_gpu, w_ref, what=what)
        return ids_ref, w_ref, np.ones(spec.T, bool)
    lg_ref = oracle.router_logits(inp["x"], inp["Wr"])
    lg_gpu = np.asarray(lg_gpu)
    dl = np.abs(lg_gpu.astype(np.float64) - lg_ref)
    bnd = logit_bound(lg_ref)
    log("%s router logits: max |diff| = %.3e, max |diff| / bound = %.3f"
        % (what, dl.max(), (dl / bnd).max()))
    assert np.all(dl <= bnd), (what, float((dl - bnd).max()))
    ids_rep, w_rep = oracle.route(lg_gpu, k)
    np.testing.assert_array_equal(ids_gpu, ids_rep)
    assert_weights_ulp(w_gpu, w_rep, what=what + " (replayed on the device's logits)")
    ids_ref, w_ref = oracle.route(lg_ref, k)
    flip = (ids_gpu != ids_ref).any(1)
    if flip.any():
        srt = -np.sort(-lg_ref.astype(np.float64), axis=1)[:, :k + 1]
        margin = (srt[:, :-1] - srt[:, 1:]).min(1)
        assert np.all(margin[flip] <= 2 * bnd.max()), (what, np.flatnonzero(flip))
    log("%s: %d near-tie tokens route differently from the oracle's own logits"
        % (what, int(flip.sum())))
    keep = ~flip
    extra = 2.0 * w_ref[keep].astype(np.float64) * dl[keep].max(1, keepdims=True)
    assert_weights_ulp(w_gpu[keep], w_ref[keep], extra=extra, what=what + " (own logits)")
    return ids_ref, w_ref, keep


def targeted_rows(offsets: np.ndarray, tile_rows=(256,), small: int = 16) -> np.ndarray:
    """Rows of the expert-sorted order that exercise the edges of the grouped GEMMs: the first and
    last row of every non-empty expert, the first and last row of every row tile of each height
    in tile_rows (a tile never straddles two experts; the last one of an expert is ragged), and
    every row of experts with fewer than ``small`` rows. A K-cut tile covers whole rows of one row
    tile, so its rows are among these."""
    rows = set()
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        m = hi - lo
        if m == 0:
            continue
        rows.update((lo, hi - 1))
        if m < small:
            rows.update(range(lo, hi))
        for bm in tile_rows:
            for r0 in range(lo, hi, bm):
                rows.update((r0, min(r0 + bm, hi) - 1))
    return np.array(sorted(rows), np.int64)


def targeted_tokens(offsets, sorted_pair, k, tile_rows=(256,), small=16, n_random=24, seed=0,
                    T=None):
    """Tokens owning the targeted rows, plus n_random random tokens (sorted, unique)."""
    rows = targeted_rows(offsets, tile_rows, small)
    toks = set((np.asarray(sorted_pair)[rows] // k).tolist())
    if n_random and T:
        rng = np.random.default_rng(seed)
        toks.update(rng.choice(T, min(n_random, T), replace=False).tolist())
        toks.update((0, T - 1))
    return np.array(sorted(toks), np.int64)


def check_edge_rows_permuted(spec, x, logits, W, S, ex_sub, remap, tile_rows, rel, what,
                             scale_fmt="f32", w_fp4=False):
    """The grouped GEMMs' edge rows of a full-size low-precision layer, per (token, expert) pair.

    Runs route -> permute -> activation quantisation -> experts with the unweighted, sorted-order
    output layout (the same GEMM kernels and tile schedule as the benchmarked slot layout; only the
    store of the down epilogue differs), then compares the targeted rows (targeted_rows) of the
    experts the oracle holds (``remap``: expert id -> index in ex_sub) with the oracle's per-pair
    expert outputs. Returns the number of rows compared."""
    import mixture_experts_ffn_softmax_amd as moe
    k = spec.k
    xd = to_dev(x)
    ids, w, _ = moe.moe_route(k, logits=to_dev(logits))
    perm = moe.moe_permute(ids, spec.E)
    xq, xs = moe.fp8_quantize_act(xd, scale_fmt=scale_fmt)
    y = moe.moe_experts_forward(xq, W[0], W[1], W[2], perm.offsets, perm.sorted_pair, w, k,
                                y_layout="permuted", x_scales=xs, s_gate=S[0], s_up=S[1],
                                s_down=S[2], scale_fmt=scale_fmt, w_fp4=w_fp4)
    torch.cuda.synchronize()
    offsets, sp = to_host(perm.offsets), to_host(perm.sorted_pair)
    ids_h = to_host(ids).reshape(-1)
    rows = targeted_rows(offsets, tile_rows)
    rows = np.array([r for r in rows if int(ids_h[sp[r]]) in remap], np.int64)
    tok = (sp[rows] // k).astype(np.int32)
    exp_sub = np.array([remap[int(ids_h[sp[r]])] for r in rows], np.int32)
    _, y_ref = oracle.expert_pairs(x, ex_sub, tok, exp_sub, want_h=False)
    got = out_to_f64(y)[rows]
    assert np.all(np.isfinite(got))
    assert_close_rel_max(got, y_ref, rel, "%s edge rows (%d pairs)" % (what, rows.size))
    return rows.size
