"""gdn_chunk_fwd_noalloc -- the chunk path on the library's static device scratch instead of a
caller workspace -- against gdn_chunk_fwd, both through the C ABI: three calls in a row on one
process's scratch, each smaller than the one before, each bitwise equal to gdn_chunk_fwd on the same
inputs (the same kernels run; only the workspace address differs) and within the oracle's
tolerances."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_amd as gdn
import gdn_inputs as gi
from tests.gpu_util import check, dev_inputs, run_oracle, say

pytestmark = pytest.mark.gpu


def _run_both(x):
    d = dev_inputs(x)
    cu_h = torch.from_numpy(x.cu.astype(np.int64))
    T, N, Hv = int(x.cu[-1]), len(x.cu) - 1, int(x.v.shape[1])
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], d["h0"])
    o_ref, h_ref = gdn.gdn_chunk_fwd(*args, cu_seqlens_host=cu_h)
    o = torch.full((T, Hv, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    hT = torch.full((N, Hv, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_chunk_fwd_noalloc(*args, o=o, hT=hT, cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    return o, hT, o_ref, h_ref


def test_noalloc_equals_workspace_entry_point():
    cases = [
        # the largest shape the scratch holds at Hv = 32: 110 record slots of 32 v-heads
        ("max: T=7039 Hk=16 Hv=32", gi.make_gdn_inputs(16, 32, [7039], seed=500)),
        # one sequence at Hv = 4: the time split, which also uses the scratch's state buffers
        ("split: T=3000 Hk=2 Hv=4 h0", gi.make_gdn_inputs(2, 4, [3000], seed=501, with_h0=True)),
        # a smaller batch over the earlier calls' leftovers, with an empty sequence
        ("varlen: [300, 0, 400] Hk=2 Hv=8 h0", gi.make_gdn_inputs(2, 8, [300, 0, 400], seed=502, with_h0=True)),
    ]
    sizes = [gdn.gdn_chunk_fwd_workspace_size(int(x.cu[-1]), len(x.cu) - 1, x.q.shape[1], x.v.shape[1])
             for _, x in cases]
    assert sizes[0] <= gdn.NOALLOC_SCRATCH_BYTES and sizes[0] > sizes[1] > sizes[2]
    for tag, x in cases:
        say(f"[noalloc] {tag}")
        o, hT, o_ref, h_ref = _run_both(x)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "o differs from gdn_chunk_fwd"
        assert torch.equal(hT, h_ref), "hT differs from gdn_chunk_fwd"
        check(o.float().cpu().numpy().astype(np.float64), hT.cpu().numpy().astype(np.float64), *run_oracle(x),
              tag)


def test_noalloc_rejects_shapes_past_the_scratch():
    x = gi.make_gdn_inputs(16, 32, [7040], seed=503)
    d = dev_inputs(x)
    o = torch.empty((7040, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], None, o=o,
                                  cu_seqlens_host=torch.from_numpy(x.cu.astype(np.int64)))
    assert e.value.code == gdn.GDN_ERR_SCRATCH_LIMIT
