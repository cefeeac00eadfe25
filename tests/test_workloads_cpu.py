"""CPU checks of the synthetic workloads' stated structure (no GPU)."""
import numpy as np

from dropless_moe_dispatch_amd import synth
from oracle import moe_oracle as O

# the skewed workload's named outcome: a few experts above 10% of the
# assignments, several with 0 or fewer than 16 rows
FEW_HOT, HOT_SHARE = 2, 0.10
SEVERAL_COLD, COLD_ROWS = 3, 16


def _skew(counts):
    share = counts / counts.sum()
    return int((share > HOT_SHARE).sum()), int((counts < COLD_ROWS).sum())


def test_skewed_workload_draw_is_the_first_with_the_named_skew():
    """The oracle's routing of the skewed workload (its own logits rounded to
    fp32, top-K on them) under each draw of the Zipf permutation stream: the
    workload's draw is the first that shows the named outcome."""
    wl = synth.WORKLOADS[5]
    inp = synth.make_inputs(wl, tensors=("x", "wg"))
    z = O.router_logits(inp["x"], inp["wg"], None)
    first = None
    for draw in range(wl.zipf_draw + 1):
        b = synth.zipf_bias(wl.seed, wl.E, wl.zipf_s, draw).astype(np.float64)
        ids = O.topk_select((z + b[None, :]).astype(np.float32), wl.K)
        hot, cold = _skew(np.bincount(ids.reshape(-1), minlength=wl.E))
        if hot >= FEW_HOT and cold >= SEVERAL_COLD:
            first = draw
            break
    assert first == wl.zipf_draw, (first, wl.zipf_draw)
    assert np.array_equal(inp["bias"], synth.zipf_bias(wl.seed, wl.E, wl.zipf_s, wl.zipf_draw))


def test_zipf_bias_is_a_log_zipf_profile_over_a_permutation():
    b = synth.zipf_bias(7, 64, 1.2, 3).astype(np.float64)
    r = np.exp(-b / 1.2)
    np.testing.assert_allclose(np.sort(r), np.arange(1, 65), rtol=1e-5)
    assert not np.array_equal(b, synth.zipf_bias(7, 64, 1.2, 0))
