"""The time split of one long sequence with few v-heads (at most 8, at least 32 chunks): the state
pass runs over 4 or more segments at once (end states from zero states, transitions from the
identity with v = 0, a scan, then the outputs from each segment's true initial state).  Parity
with the fp64 oracle to the usual tolerances, and the properties that still hold bitwise: the two
stages called separately equal one call, an in-place final state equals a separate one, and an
indexed initial state equals the same state passed directly."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_amd as gdn
import gdn_inputs as gi
from tests.gpu_util import check, dev_inputs, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("Hk,Hv,T,with_h0,g_mean", [
    (1, 2, 2100, True, 3.0),     # 33 chunks: 4 segments of 9, 6 the last; ragged last chunk
    (2, 4, 4133, False, 3.0),    # 65 chunks: 8 segments of 9, 2 the last
    (4, 8, 2048, True, 6.0),     # 32 chunks: 4 segments of 8; slow decay, h0 felt throughout
])
def test_split_parity(Hk, Hv, T, with_h0, g_mean):
    say(f"[split] Hk={Hk} Hv={Hv} T={T} h0={with_h0} g_mean={g_mean}")
    x = gi.make_gdn_inputs(Hk, Hv, [T], seed=300 + T % 97, with_h0=with_h0, g_mean=g_mean)
    o, hT = run_gpu(x)
    check(o, hT, *run_oracle(x), f"split T={T}")


def _plan(x, **kw):
    d = dev_inputs(x)
    return gdn.ChunkPlan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], d["h0"],
                         cu_seqlens_host=torch.from_numpy(x.cu.astype(np.int64)), **kw), d


def test_split_stages_equal_one_call():
    say("[split-stages] Hk=2 Hv=4 T=3000 h0: prep + pass vs one call")
    x = gi.make_gdn_inputs(2, 4, [3000], seed=310, with_h0=True)
    p1, _ = _plan(x)
    p1.forward()
    p2, _ = _plan(x)
    p2.prep()
    p2.state_pass()
    torch.cuda.synchronize()
    assert torch.equal(p1.o.view(torch.int16), p2.o.view(torch.int16)) and torch.equal(p1.hT, p2.hT)


def test_split_in_place_and_indexed():
    say("[split-state-args] Hk=1 Hv=4 T=2500: hT aliasing h0, and h0 from a pool by index")
    x = gi.make_gdn_inputs(1, 4, [2500], seed=320, with_h0=True)
    d = dev_inputs(x)
    cu_h = torch.from_numpy(x.cu.astype(np.int64))
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    o1, h1 = gdn.gdn_chunk_fwd(*args, d["h0"].clone(), cu_seqlens_host=cu_h)
    buf = d["h0"].clone()
    o2, h2 = gdn.gdn_chunk_fwd(*args, buf, hT=buf, cu_seqlens_host=cu_h)
    pool = torch.stack([torch.zeros_like(d["h0"][0]), d["h0"][0]])
    o3, h3 = gdn.gdn_chunk_fwd_indexed(*args, pool, torch.tensor([1], dtype=torch.int32, device="cuda"),
                                       cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    assert h2.data_ptr() == buf.data_ptr()
    for o_, h_ in ((o2, h2), (o3, h3)):
        assert torch.equal(o_.view(torch.int16), o1.view(torch.int16)) and torch.equal(h_, h1)
    check(o1.float().cpu().numpy().astype(np.float64), h1.cpu().numpy().astype(np.float64), *run_oracle(x),
          "split with h0")
