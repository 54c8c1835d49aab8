"""gdn_chunk_fwd and gdn_mixer_fwd (HIP) against the fp64 oracles over seeded sweeps of shapes: numbers of sequences,
mixes of lengths (empty, a few tokens, around a chunk boundary, several chunks), head counts and
k/v head ratios, with and without initial states.  The cases reach the single-round and the
persistent state pass, the time split of one long sequence, and both forms of the chunk prep (two
v-heads per workgroup, or one when a k-head has an odd number of v-heads).  Same bars as the other
parity tests (o rel-L2 5e-3, max-abs 2e-2; hT rel-L2 1e-3; for the mixer, y as in test_gpu_mixer)."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_deltanet_chunked_amd as gdn
import gdn_inputs as gi
import oracle
from tests.gpu_util import bf16_dev, check, f32_dev, run_gpu, run_oracle, say
from tests.test_gpu_mixer import check_mixer, run_mixer_gpu, run_mixer_oracle

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


def _mixer_cases(count=8, seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        Hk = int(rng.choice([1, 2, 4, 8, 16]))
        r = int(rng.choice([1, 2, 3, 4]))
        while Hk * r > 32:
            r -= 1
        N = int(rng.integers(1, 9))
        lengths = [_length(rng) for _ in range(N)]
        if sum(lengths) == 0:
            lengths[0] = 1
        out.append((i, Hk, Hk * r, lengths, bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("i,Hk,Hv,lengths,with_h0", _mixer_cases(), ids=lambda v: None)
def test_random_mixer_shapes(i, Hk, Hv, lengths, with_h0):
    # gdn_mixer_fwd, and on even cases gdn_mixer_fwd_gates (gates made in the first kernel, against
    # the oracle's fp64 gates): odd head ratios run the separate input prep, even ones the chunk
    # prep that makes q, k, v itself; zero-length and few-token sequences reset the conv window.
    say(f"[mixer sweep {i}] Hk={Hk} Hv={Hv} N={len(lengths)} T={sum(lengths)} h0={with_h0} lengths={lengths}")
    m = gi.make_mixer_inputs(4000 + i, lengths=lengths, Hk=Hk, Hv=Hv, with_h0=with_h0)
    check_mixer(*run_mixer_gpu(m, Hk, Hv), *run_mixer_oracle(m, Hk, Hv), f"mixer sweep {i}", m)
    if i % 2 == 0:
        gt = gi.make_gate_inputs(4100 + i, m.qkv.shape[0], Hv)
        f = gi.bits_to_f64
        g, beta = oracle.gates(f(gt.a), f(gt.b), gt.A_log.astype(np.float64), gt.dt_bias.astype(np.float64))
        y, hT = gdn.gdn_mixer_fwd_gates(bf16_dev(m.qkv), bf16_dev(m.conv_w), bf16_dev(gt.a), bf16_dev(gt.b),
                                        f32_dev(gt.A_log), f32_dev(gt.dt_bias), bf16_dev(m.z), bf16_dev(m.norm_w),
                                        torch.from_numpy(m.cu.astype(np.int32)).cuda(),
                                        None if m.h0 is None else f32_dev(m.h0), Hk=Hk, Hv=Hv,
                                        cu_seqlens_host=torch.from_numpy(m.cu.astype(np.int64)))
        torch.cuda.synchronize()
        mg = dataclasses.replace(m, g=g, beta=beta)
        check_mixer(y.float().cpu().numpy().astype(np.float64), hT.cpu().numpy().astype(np.float64),
                    *run_mixer_oracle(mg, Hk, Hv), f"mixer sweep {i} gates", mg)
