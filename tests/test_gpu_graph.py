"""HIP graph capture of the small-batch path (a serving loop replays one captured decode step).

The library enqueues only kernels on the caller's stream (no memset nodes, no allocation, no
synchronisation), so a step captured with torch.cuda.graph replays it. Each case captures once,
then replays several times with eager work and synchronisations between the replays, new inputs
copied into the captured input buffers, and checks every replay bit-exactly against the eager
result on the same inputs.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_softmax_amd as moe
import synth
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

SPEC = synth.MIXTRAL_DECODE.with_(name="graph_T32_d512_f384_E8_k2", T=32, d=512, f=384, E=8, k=2)


def _inputs(seed_shift):
    spec = SPEC.with_(x_seed=SPEC.x_seed + seed_shift)
    return to_dev(synth.gen_x(spec))


@pytest.mark.parametrize("fused", (True, False), ids=("fused", "separate"))
def test_graph_replays_match_eager(fused):
    log("graph capture", "fused" if fused else "separate calls")
    W = [to_dev(synth.gen_expert_weight(SPEC, n)) for n in ("gate", "up", "down")]
    wr = to_dev(synth.gen_router_weight(SPEC))
    x_buf = _inputs(0).clone()

    def step():
        if fused:
            out, ids, _ = moe.moe_fused_forward(x_buf, *W, SPEC.k, w_router=wr)
        else:
            res = moe.moe_layer(x_buf, *W, SPEC.k, w_router=wr)
            out, ids = res.out, res.topk_ids
        return out, ids

    step()                                   # warm-up outside capture (library load, caches)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g):
            out_g, ids_g = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        x_buf.copy_(_inputs(rep + 1))
        eager_out, eager_ids = step()        # eager work between the replays
        eager_out, eager_ids = eager_out.clone(), eager_ids.clone()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids_g, eager_ids), "replay %d: routing differs" % rep
        assert torch.equal(out_g, eager_out), "replay %d: output differs" % rep
    assert torch.isfinite(out_g.float()).all()
