"""moe_fused_forward_noalloc against moe_fused_forward, through the C ABI.

The allocation-free variant runs the fused small-batch path with the library's own device scratch
array in place of a caller's workspace; it must give bit-identical outputs, routing ids and
weights (same kernels, same arithmetic). Two calls in a row, the second on a smaller batch, so
that the second call runs on the array the first one left behind; the reference calls use a
garbage-filled workspace of their own.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_softmax_amd as moe
import synth
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def _weights(spec, fmt):
    W = [to_dev(synth.gen_expert_weight(spec, n)) for n in ("gate", "up", "down")]
    if fmt == "bf16":
        return W, [None] * 3
    if fmt == "fp4":
        pairs = [moe.fp4_quantize_weight_mx(w.float(), tiled=True) for w in W]
    else:
        pairs = [moe.fp8_quantize_weight(w.float(), scale_fmt=fmt) for w in W]
    return [q for q, _ in pairs], [s for _, s in pairs]


def _reference(spec, x, W, S, wr, fmt):
    n = moe.load_library().moe_fused_workspace_size(
        spec.T, spec.d, spec.f, spec.E, spec.k,
        {"bf16": moe.MOE_BF16, "fp4": moe.MOE_FP4_E2M1}.get(fmt, moe.MOE_FP8_E4M3), moe.MOE_BF16)
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    return moe.moe_fused_forward(x, *W, spec.k, w_router=wr, s_gate=S[0], s_up=S[1], s_down=S[2],
                                 w_fp4=fmt == "fp4", workspace=ws)


@pytest.mark.parametrize("fmt", ("bf16", "ue8m0", "f32", "fp4"))
def test_noalloc_matches_workspace_call(fmt):
    big = synth.MIXTRAL_DECODE.with_(name="noalloc_T32_d1024_f2048_E8_k2", T=32, d=1024, f=2048)
    small = big.with_(name="noalloc_T5", T=5)
    W, S = _weights(big, fmt)
    wr = to_dev(synth.gen_router_weight(big))
    for spec in (big, small):
        log("noalloc", fmt, spec.name)
        x = to_dev(synth.gen_x(spec))
        ref = _reference(spec, x, W, S, wr, fmt)
        out = torch.empty((spec.T, spec.d), dtype=torch.bfloat16, device="cuda")
        ids = torch.empty((spec.T, spec.k), dtype=torch.int32, device="cuda")
        w = torch.empty((spec.T, spec.k), dtype=torch.float32, device="cuda")
        got = moe.moe_fused_forward(x, *W, spec.k, w_router=wr, s_gate=S[0], s_up=S[1],
                                    s_down=S[2], w_fp4=fmt == "fp4", noalloc=True, out=out,
                                    topk_ids=ids, topk_w=w)
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("out", "topk_ids", "topk_w")):
            assert torch.equal(a, b), (fmt, spec.name, name)
        assert torch.isfinite(got[0].float()).all()


def test_noalloc_mixtral_decode_full_size():
    # the Mixtral-shaped decode layer (d = 4096, f = 14336) with bf16 experts, then a smaller batch
    spec = synth.MIXTRAL_DECODE
    W, S = _weights(spec, "bf16")
    wr = to_dev(synth.gen_router_weight(spec))
    for T in (spec.T, 3):
        s = spec.with_(T=T)
        log("noalloc mixtral decode T=%d" % T)
        x = to_dev(synth.gen_x(s))
        ref = _reference(s, x, W, S, wr, "bf16")
        got = moe.moe_fused_forward(x, *W, s.k, w_router=wr, noalloc=True)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
