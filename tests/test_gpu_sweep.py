"""gdn_chunk_fwd (HIP) against the fp64 oracle over a seeded sweep of shapes: numbers of sequences,
mixes of lengths (empty, a few tokens, around a chunk boundary, several chunks), head counts and
k/v head ratios, with and without initial states.  The cases reach the single-round and the
persistent state pass, the time split of one long sequence, and both forms of the chunk prep (two
v-heads per workgroup, or one when a k-head has an odd number of v-heads).  Same bars as the other
parity tests (o rel-L2 5e-3, max-abs 2e-2; hT rel-L2 1e-3)."""
import numpy as np
import pytest

import gdn_inputs as gi
from tests.gpu_util import check, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


def _length(rng):
    u = rng.random()
    if u < 0.1:
        return 0
    if u < 0.25:
        return int(rng.integers(1, 4))
    if u < 0.45:
        return int(rng.integers(60, 70))
    return int(rng.integers(1, 400))


def _cases(count=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        Hk = int(rng.choice([1, 2, 4, 8, 16]))
        r = int(rng.choice([1, 2, 3, 4]))
        while Hk * r > 64:
            r -= 1
        Hv = Hk * r
        if i % 5 == 4 and Hv <= 8:
            lengths = [int(rng.integers(2000, 4000))]  # one long sequence: the time split
        else:
            N = int(rng.integers(1, 13))
            lengths = [_length(rng) for _ in range(N)]
            if sum(lengths) == 0:
                lengths[0] = 1
        out.append((i, Hk, Hv, lengths, bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("i,Hk,Hv,lengths,with_h0", _cases(), ids=lambda v: None)
def test_random_shapes(i, Hk, Hv, lengths, with_h0):
    say(f"[sweep {i}] Hk={Hk} Hv={Hv} N={len(lengths)} T={sum(lengths)} h0={with_h0} lengths={lengths}")
    x = gi.make_gdn_inputs(Hk, Hv, lengths, seed=3000 + i, with_h0=with_h0)
    o, hT = run_gpu(x)
    o_ref, h_ref = run_oracle(x)
    check(o, hT, o_ref, h_ref, f"sweep {i}")
