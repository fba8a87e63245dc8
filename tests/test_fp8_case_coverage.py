"""The skewed fp8 parity cases reach the tile kinds their comments name (CPU check of the inputs).

The tiled fp8 GEMMs with UE8M0 scales split each expert's rows into 256-row blocks: a block of
more than 128 rows runs as one 256-row tile (8 waves of 64 rows; a wave whose rows all lie past
the block's last row idles), a shorter block as a 128-row tile. The GPU cases in
test_gpu_fp8.SMALL are only worth their run time if the oracle's routing of their seeded logits
actually produces each kind; this pins that, so a change to the generator or the specs that loses
one fails here rather than silently thinning the GPU coverage."""
import numpy as np

import oracle
import synth
from test_gpu_fp8 import SMALL


def _blocks(counts):
    """(rows of every 256-row block) over all experts."""
    out = []
    for m in counts:
        for r0 in range(0, int(m), 256):
            out.append(min(256, int(m) - r0))
    return out


def test_skewed_fp8_cases_cover_every_tile_kind():
    blocks, counts_all, stages = [], [], set()
    for spec in SMALL:
        if not spec.name.startswith("fp8_skew"):
            continue
        ids, _ = oracle.route(synth.gen_logits(spec), spec.k)
        counts = np.bincount(ids.reshape(-1), minlength=spec.E)
        counts_all += counts.tolist()
        blocks += _blocks(counts)
        stages.update({spec.d // 128 % 2, spec.f // 128 % 2})   # K stages of gate/up and down
    assert any(b == 256 for b in blocks), "a full 256-row tile"
    assert any(128 < b < 256 and b <= 192 for b in blocks), "a 256-row tile whose last wave row idles"
    assert any(192 < b < 256 for b in blocks), "a ragged 256-row tile with every wave row active"
    assert any(b <= 64 and m > 256 for m in counts_all for b in _blocks([m])[-1:]), \
        "a remainder past 256 rows that fills one wave row"
    assert any(64 < b <= 128 and m > 256 for m in counts_all for b in _blocks([m])[-1:]), \
        "a remainder past 256 rows that fills two wave rows"
    assert any(0 < m <= 128 for m in counts_all), "an expert that is one 128-row tile"
    assert any(m > 512 for m in counts_all), "an expert of more than two 256-row blocks"
    assert stages == {0, 1}, "odd and even stage counts"
