"""moe_build_index_noalloc (the index without a caller workspace, for callers
that cannot allocate) against moe_build_index through the C-ABI: two calls in
a row, the second with a smaller input, each bit-exact against the
workspace entry point on the same ids (and the oracle's index of them)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from dropless_moe_dispatch_amd import binding as B
from dropless_moe_dispatch_amd import layer as Lyr
from dropless_moe_dispatch_amd import synth
from oracle import moe_oracle as O
from tests.gpu_util import to_np

pytestmark = pytest.mark.gpu


def _index_both(T, E, K, kind, seed):
    print("[case] noalloc index", T, E, K, kind, file=sys.stderr, flush=True)
    z = synth.structured_logits(T, E, K, kind, seed=seed)
    ids = O.topk_select(z, K)
    ref = Lyr.MoEBuffers(T, 128, E, K, 128, "bf16", backward=False)
    got = Lyr.MoEBuffers(T, 128, E, K, 128, "bf16", backward=False)
    ref.topk_ids.copy_(torch.from_numpy(ids))
    got.topk_ids.copy_(torch.from_numpy(ids))
    for t in (got.offsets, got.eti, got.tim):
        t.fill_(-7)                          # every output element must be written
    B.moe_build_index(ref.shape, ref.topk_ids, ref.offsets, ref.eti, ref.tim, ref.ws_index)
    B.moe_build_index_noalloc(got.shape, got.topk_ids, got.offsets, got.eti, got.tim)
    torch.cuda.synchronize()
    for k in ("offsets", "eti", "tim"):
        assert torch.equal(getattr(got, k), getattr(ref, k)), k
    ix = O.build_index(ids, E)
    assert np.array_equal(to_np(got.offsets), ix["offsets"])
    assert np.array_equal(to_np(got.eti), ix["expert_token_indices"])
    assert np.array_equal(to_np(got.tim), ix["token_index_map"])


def test_noalloc_index_matches_the_workspace_entry_point_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    # the first call fills much of the static scratch; the second, smaller one
    # runs over what it left there
    _index_both(20000, 1000, 8, "gaussian", seed=3)
    _index_both(300, 16, 4, "zero_rows", seed=4)


def test_noalloc_index_refuses_shapes_past_its_scratch():
    s = B.shape(65536, 128, 1024, 8, 128)
    assert B.workspace_bytes(s, B.MOE_WS_INDEX) > 8 << 20
    fake = 0x10000
    rc = B.moe_build_index_noalloc(s, fake, fake, fake, fake, stream=0, check=False)
    assert rc == B.MOE_ERR_WORKSPACE
