"""gdn_chunk_fwd with token offsets past 2**31 bytes (v and o rows beyond 262,144 tokens at Hv = 32):
every byte offset in the kernels is 64-bit.  Inputs are drawn on the GPU (seeded torch generator,
the distributions of the benchmark workloads) because the host draw of ~9 GB would take minutes;
the oracle sees exactly the same values, copied back.

* A packed batch [L0, 300] with L0 = 270,037: the second sequence starts past the 2**31-byte
  mark; its outputs and final state, and the first 300 outputs of the long sequence, against the
  fp64 oracle.
* The long sequence alone (one-round grid) equals its packed run bitwise (packed-batch grid).
* The long sequence split at a chunk boundary near its end and continued from its own state
  equals one run bitwise: the tail computed at large offsets matches the tail computed at small
  ones."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_amd as gdn
import gdn_inputs as gi
from tests.gpu_util import check, run_oracle, say

pytestmark = pytest.mark.gpu

HK, HV, D = 16, 32, 128
L0, L1 = 270_037, 300


def _draw(T, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)

    def unit(h):
        x = torch.randn((T, h, D), generator=gen, device="cuda", dtype=torch.float32)
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    q, k = unit(HK), unit(HK)
    v = torch.randn((T, HV, D), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn((T, HV), generator=gen, device="cuda"))
    g = torch.nn.functional.logsigmoid(3.0 + torch.randn((T, HV), generator=gen, device="cuda"))
    return q, k, v, g.contiguous(), beta.contiguous()


def _host(q, k, v, g, beta, lo, hi):
    bits = lambda t: t[lo:hi].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return gi.GdnInputs(bits(q), bits(k), bits(v), beta[lo:hi].cpu().numpy(), g[lo:hi].cpu().numpy(),
                        np.array([0, hi - lo], np.int32), None)


def _run(q, k, v, g, beta, lengths, h0=None):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    o, hT = gdn.gdn_chunk_fwd(q, k, v, g, beta, torch.from_numpy(cu.astype(np.int32)).cuda(), h0,
                              cu_seqlens_host=torch.from_numpy(cu))
    torch.cuda.synchronize()
    return o, hT


def test_offsets_past_2gib():
    T = L0 + L1
    say(f"[large] T={T} (lengths {L0}, {L1}) Hk={HK} Hv={HV}: v and o span {T * HV * D * 2 / 2**30:.2f} GiB")
    q, k, v, g, beta = _draw(T, 7)
    o, hT = _run(q, k, v, g, beta, [L0, L1])
    assert L0 * HV * D * 2 > 2 ** 31

    # the sequence that starts past 2 GiB (outputs and final state) against the oracle
    o_ref, h_ref = run_oracle(_host(q, k, v, g, beta, L0, T))
    check(o[L0:T].float().cpu().numpy().astype(np.float64), hT[1:2].cpu().numpy().astype(np.float64),
          o_ref, h_ref, f"sequence 1, tokens {L0}..{T}")
    # the first L1 outputs of the long sequence (its state there is internal: o only)
    o_ref, h_ref = run_oracle(_host(q, k, v, g, beta, 0, L1))
    check(o[:L1].float().cpu().numpy().astype(np.float64), h_ref, o_ref, h_ref, f"sequence 0, tokens 0..{L1}")

    # the long sequence alone (one workgroup per item) equals its packed run
    o0, h0_ = _run(q[:L0], k[:L0], v[:L0], g[:L0], beta[:L0], [L0])
    assert torch.equal(o0.view(torch.int16), o[:L0].view(torch.int16)), "long sequence: o differs from packed run"
    assert torch.equal(h0_[0], hT[0]), "long sequence: state differs from packed run"
    del o0

    # split near the end at a chunk boundary, continued from its own state: bitwise
    T1 = (L0 - 320) // 64 * 64
    _, ha = _run(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], [T1])
    ob, hb = _run(q[T1:L0], k[T1:L0], v[T1:L0], g[T1:L0], beta[T1:L0], [L0 - T1], h0=ha)
    say(f"  split at {T1}: tail of {L0 - T1} tokens from byte offset {T1 * HV * D * 2 / 2**30:.2f} GiB")
    assert torch.equal(ob.view(torch.int16), o[T1:L0].view(torch.int16)), "tail differs from one run"
    assert torch.equal(hb[0], hT[0]), "final state differs from one run"
