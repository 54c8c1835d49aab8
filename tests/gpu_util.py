"""Helpers for the GPU tests: move seeded inputs to the device, run the oracle, compare."""
import sys

import numpy as np
import torch

import gated_deltanet_chunked_amd as gdn
import gdn_inputs as gi
import oracle

# Tolerances for gdn_chunk_fwd against the fp64 oracle (o is bf16, hT is fp32).
O_REL, O_ABS, H_REL = 5e-3, 2e-2, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def f32_dev(x, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def dev_inputs(x: gi.GdnInputs, dev="cuda"):
    return dict(q=bf16_dev(x.q, dev), k=bf16_dev(x.k, dev), v=bf16_dev(x.v, dev), g=f32_dev(x.g, dev),
                beta=f32_dev(x.beta, dev), cu=torch.from_numpy(x.cu.astype(np.int32)).to(dev),
                h0=None if x.h0 is None else f32_dev(x.h0, dev))


def run_gpu(x: gi.GdnInputs, dev="cuda", **kw):
    d = dev_inputs(x, dev)
    o, hT = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], d["h0"],
                              cu_seqlens_host=torch.from_numpy(x.cu.astype(np.int64)), **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), (None if hT is None else hT.cpu().numpy().astype(np.float64))


def run_oracle(x: gi.GdnInputs):
    q, k, v, g, b, cu, h0 = x.f64()
    return oracle.gdn_fwd(q, k, v, g, b, cu, h0)


def rel_l2(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


def check(o, hT, o_ref, h_ref, tag=""):
    ro, mo = rel_l2(o, o_ref), float(np.abs(o - o_ref).max()) if o.size else 0.0
    rh = rel_l2(hT, h_ref)
    say(f"  {tag}: o rel-L2 {ro:.3e} max-abs {mo:.3e} | hT rel-L2 {rh:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT)), "non-finite output"
    assert ro <= O_REL, f"o rel-L2 {ro}"
    assert mo <= O_ABS, f"o max-abs {mo}"
    assert rh <= H_REL, f"hT rel-L2 {rh}"
    return ro, mo, rh
