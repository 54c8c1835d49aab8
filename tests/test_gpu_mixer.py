"""gdn_mixer_fwd (HIP) against the fp64 mixer oracle: y rel-L2 <= 5e-3, an elementwise bound on y
propagated from the 2e-2 max-abs tolerance of o through the gated RMSNorm (see check_mixer), and
hT rel-L2 <= 1e-3."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_deltanet_chunked_amd as gdn
import gdn_inputs as gi
import oracle
from tests.gpu_util import bf16_dev, f32_dev, rel_l2, say

pytestmark = pytest.mark.gpu


def run_mixer_gpu(m: gi.MixerInputs, Hk=16, Hv=32, fused_norm=False):
    y, hT = gdn.gdn_mixer_fwd(bf16_dev(m.qkv), bf16_dev(m.conv_w), f32_dev(m.g), f32_dev(m.beta), bf16_dev(m.z),
                              bf16_dev(m.norm_w), torch.from_numpy(m.cu.astype(np.int32)).cuda(),
                              None if m.h0 is None else f32_dev(m.h0), Hk=Hk, Hv=Hv,
                              cu_seqlens_host=torch.from_numpy(m.cu.astype(np.int64)), fused_norm=fused_norm)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), hT.cpu().numpy().astype(np.float64)


def run_mixer_oracle(m: gi.MixerInputs, Hk=16, Hv=32):
    """(y, hT, o) from the fp64 oracle.  o, the rule's output at its bf16 rounding point, is not an
    output of the mixer, so it is rebuilt from the oracle's pieces (conv + SiLU, L2 norm, bf16
    rounding points, the rule); it only sets the scale of the elementwise bound on y."""
    f = gi.bits_to_f64
    h0 = None if m.h0 is None else m.h0.astype(np.float64)
    y, hT = oracle.mixer_fwd(f(m.qkv), f(m.conv_w), m.g.astype(np.float64), m.beta.astype(np.float64), f(m.z),
                             f(m.norm_w), m.cu.astype(np.int64), h0, Hk=Hk, Hv=Hv)
    T, d = m.qkv.shape[0], 128
    a = oracle.conv_silu(f(m.qkv), f(m.conv_w), m.cu.astype(np.int64))
    l2 = lambda x: x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)
    q = oracle.round_bf16(l2(a[:, :Hk * d].reshape(T, Hk, d)))
    k = oracle.round_bf16(l2(a[:, Hk * d:2 * Hk * d].reshape(T, Hk, d)))
    v = oracle.round_bf16(a[:, 2 * Hk * d:].reshape(T, Hv, d))
    o, _ = oracle.gdn_fwd(q, k, v, m.g, m.beta, m.cu, h0)
    return y, hT, oracle.round_bf16(o)


def check_mixer(y, hT, y_ref, h_ref, o_ref, tag, m: gi.MixerInputs):
    """Mixer tolerance, derived from the gdn_chunk_fwd tolerance on o.

    y = o r c with r = 1 / rms(o_row) and c = w silu(z).  An absolute error e in o becomes
    c r (e - o (o.e) / (d rms^2)) in y, at most |c| r |e|max (1 + |o| / rms); the bf16 output adds
    at most half an ulp (2^-9 |y|).  So elementwise |dy| <= |c| r 2e-2 (1 + |o| r) + 2^-8 |y_ref|,
    with 2e-2 the max-abs tolerance of o.  Also y rel-L2 <= 5e-3 and hT rel-L2 <= 1e-3."""
    ry = rel_l2(y, y_ref)
    rh = rel_l2(hT, h_ref)
    zf = gi.bits_to_f64(m.z)
    c = np.abs(gi.bits_to_f64(m.norm_w) * zf / (1 + np.exp(-zf)))
    r = 1.0 / np.sqrt(np.mean(o_ref ** 2, axis=-1, keepdims=True) + 1e-6)
    bound = c * r * 2e-2 * (1 + np.abs(o_ref) * r) + 2.0 ** -8 * np.abs(y_ref)
    ratio = np.abs(y - y_ref) / bound
    i = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else None
    worst = float(ratio[i]) if i is not None else 0.0
    detail = "" if i is None else (f" at {i}: |dy| {abs(y[i] - y_ref[i]):.3e} y {y_ref[i]:.3e} "
                                   f"rms(o_row) {1 / r[i[0], i[1], 0]:.3e}")
    say(f"  {tag}: y rel-L2 {ry:.3e} max |dy|/bound {worst:.3f}{detail} | hT rel-L2 {rh:.3e}")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hT))
    assert ry <= 5e-3 and worst <= 1.0 and rh <= 1e-3


def pure_fp64_errors(y, hT, m: gi.MixerInputs, tag, Hk=16, Hv=32):
    """Printed, not asserted: the GPU's y and hT against the mixer in fp64 throughout, without the bf16
    rounding points of the prepped q, k, v and of o that the asserted oracle keeps (the GPU path has
    them by construction: its chunk path takes bf16 q, k, v and writes bf16 o)."""
    f = gi.bits_to_f64
    h0 = None if m.h0 is None else m.h0.astype(np.float64)
    y64, h64 = oracle.mixer_fwd(f(m.qkv), f(m.conv_w), m.g.astype(np.float64), m.beta.astype(np.float64), f(m.z),
                                f(m.norm_w), m.cu.astype(np.int64), h0, Hk=Hk, Hv=Hv, bf16_points=False)
    say(f"  {tag} vs the pure-fp64 mixer (not asserted): y rel-L2 {rel_l2(y, y64):.3e} | hT rel-L2 {rel_l2(hT, h64):.3e}")


def test_mixer_t936_layer0():
    say("[mixer] T=936 Hk=16 Hv=32 seed=100")
    m = gi.make_mixer_inputs(100)
    y, hT = run_mixer_gpu(m)
    check_mixer(y, hT, *run_mixer_oracle(m), "T=936", m)
    pure_fp64_errors(y, hT, m, "T=936")


@pytest.mark.parametrize("case", ["t936", "varlen"])
def test_mixer_fused_norm(case):
    # gdn_mixer_fwd_fused_norm: the gated RMSNorm inside the state pass.  Same tolerances as the
    # separate kernel; hT bitwise equal to gdn_mixer_fwd (the norm does not touch it); y equal up to
    # the order of the row's sum of squares.
    if case == "t936":
        m, Hk, Hv = gi.make_mixer_inputs(100), 16, 32
    else:
        m, Hk, Hv = gi.make_mixer_inputs(7, lengths=[5, 70, 3, 130, 1], Hk=2, Hv=4, with_h0=True), 2, 4
    say(f"[mixer-fused-norm] {case} Hk={Hk} Hv={Hv} T={m.qkv.shape[0]}")
    y, hT = run_mixer_gpu(m, Hk, Hv, fused_norm=True)
    y_sep, h_sep = run_mixer_gpu(m, Hk, Hv)
    assert np.array_equal(hT, h_sep), "hT differs from gdn_mixer_fwd"
    say(f"  y against gdn_mixer_fwd: rel-L2 {rel_l2(y, y_sep):.3e} max|d| {np.abs(y - y_sep).max():.3e}")
    check_mixer(y, hT, *run_mixer_oracle(m, Hk, Hv), f"fused norm {case}", m)
    pure_fp64_errors(y, hT, m, f"fused norm {case}", Hk, Hv)


@pytest.mark.parametrize("lengths,Hk,Hv", [([40] * 40, 2, 4), ([3000], 1, 4)])
def test_mixer_fused_norm_unsupported(lengths, Hk, Hv):
    # 40 sequences x 4 v-heads x 8 tiles take more than one round of workgroups; one sequence of
    # 3000 tokens at Hv = 4 takes the time split: neither is launched fused (nothing is enqueued).
    say(f"[mixer-fused-norm] unsupported: {len(lengths)} x {lengths[0]} Hk={Hk} Hv={Hv}")
    m = gi.make_mixer_inputs(9, lengths=lengths, Hk=Hk, Hv=Hv)
    with pytest.raises(gdn.GdnError) as e:
        run_mixer_gpu(m, Hk, Hv, fused_norm=True)
    assert e.value.code == gdn.GDN_ERR_UNSUPPORTED


def test_mixer_varlen_conv_resets_with_h0():
    lengths = [5, 70, 3, 130, 1]
    say(f"[mixer] varlen {lengths} Hk=2 Hv=4 with h0")
    m = gi.make_mixer_inputs(7, lengths=lengths, Hk=2, Hv=4, with_h0=True)
    check_mixer(*run_mixer_gpu(m, 2, 4), *run_mixer_oracle(m, 2, 4), "varlen", m)


def test_mixer_varlen_bitwise_equals_separate():
    lengths = [40, 3, 90]
    say(f"[mixer] varlen bitwise {lengths}")
    m = gi.make_mixer_inputs(8, lengths=lengths, Hk=2, Hv=4, with_h0=True)
    y, hT = run_mixer_gpu(m, 2, 4)
    for n, L in enumerate(lengths):
        sl = slice(m.cu[n], m.cu[n + 1])
        ms = gi.MixerInputs(m.qkv[sl], m.conv_w, m.beta[sl], m.g[sl], m.z[sl], m.norm_w,
                            np.array([0, L], np.int32), m.h0[n:n + 1])
        y1, h1 = run_mixer_gpu(ms, 2, 4)
        assert np.array_equal(y[sl], y1) and np.array_equal(hT[n], h1[0])


@pytest.mark.parametrize("Hk,Hv", [(4, 4), (1, 4), (2, 6)])
def test_mixer_head_ratios(Hk, Hv):
    # Hv / Hk odd: the input prep runs as its own kernel before the chunk prep; even: the chunk
    # prep makes q, k, v itself (with 4 v-heads per k-head, two workgroups make the same q, k and
    # the first of them writes it).
    lengths = [70, 1, 130]
    say(f"[mixer] head ratio Hk={Hk} Hv={Hv} lengths={lengths} with h0")
    m = gi.make_mixer_inputs(300 + 10 * Hk + Hv, lengths=lengths, Hk=Hk, Hv=Hv, with_h0=True)
    check_mixer(*run_mixer_gpu(m, Hk, Hv), *run_mixer_oracle(m, Hk, Hv), f"Hk={Hk} Hv={Hv}", m)


@pytest.mark.parametrize("case", ["t936", "varlen_ratio1", "varlen_ratio3", "extreme"])
def test_mixer_gates(case):
    # gdn_mixer_fwd_gates: g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b) made in the
    # mixer's first kernel (fp32 on the GPU), against the oracle's gates (fp64) fed to the mixer
    # oracle.  Ratio 2 runs them in the chunk prep that also makes q, k, v; ratios 1 and 3 in the
    # chunk prep after the separate input prep.
    if case == "t936":
        m, Hk, Hv = gi.make_mixer_inputs(100), 16, 32
    elif case == "varlen_ratio1":
        m, Hk, Hv = gi.make_mixer_inputs(11, lengths=[70, 1, 200, 33], Hk=2, Hv=2, with_h0=True), 2, 2
    elif case == "varlen_ratio3":
        m, Hk, Hv = gi.make_mixer_inputs(12, lengths=[129, 64, 5], Hk=1, Hv=3), 1, 3
    else:
        m, Hk, Hv = gi.make_mixer_inputs(13, lengths=[150, 70], Hk=2, Hv=4, with_h0=True), 2, 4
    T = m.qkv.shape[0]
    gt = gi.make_gate_inputs(200, T, Hv)
    if case == "extreme":
        # softplus far in both tails (a + dt_bias up to +-120: the decay saturates, e^g underflows
        # to zero and the state restarts; or softplus underflows and the state is kept), beta at
        # 0 and 1 (b = -+90), and decay rates A from 1e-3 to 1e3
        rng = np.random.default_rng(201)
        a = rng.choice([-120.0, -40.0, -3.0, 0.0, 3.0, 40.0, 120.0], size=(T, Hv))
        b = rng.choice([-90.0, -8.0, 0.0, 8.0, 90.0], size=(T, Hv))
        gt = gi.GateInputs(gi.bf16_bits(a), gi.bf16_bits(b),
                           np.log(np.array([1e-3, 1.0, 30.0, 1e3][:Hv])).astype(np.float32), gt.dt_bias)
    say(f"[mixer-gates] {case} Hk={Hk} Hv={Hv} T={T}")
    f = gi.bits_to_f64
    g, beta = oracle.gates(f(gt.a), f(gt.b), gt.A_log.astype(np.float64), gt.dt_bias.astype(np.float64))
    say(f"  g in [{g.min():.3f}, {g.max():.3f}], beta in [{beta.min():.3f}, {beta.max():.3f}]")
    y, hT = gdn.gdn_mixer_fwd_gates(bf16_dev(m.qkv), bf16_dev(m.conv_w), bf16_dev(gt.a), bf16_dev(gt.b),
                                    f32_dev(gt.A_log), f32_dev(gt.dt_bias), bf16_dev(m.z), bf16_dev(m.norm_w),
                                    torch.from_numpy(m.cu.astype(np.int32)).cuda(),
                                    None if m.h0 is None else f32_dev(m.h0), Hk=Hk, Hv=Hv,
                                    cu_seqlens_host=torch.from_numpy(m.cu.astype(np.int64)))
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    hT = hT.cpu().numpy().astype(np.float64)
    mg = dataclasses.replace(m, g=g, beta=beta)
    check_mixer(y, hT, *run_mixer_oracle(mg, Hk, Hv), f"gates {case}", mg)


@pytest.mark.parametrize("form", ["plain", "gates"])
def test_mixer_plan(form):
    # MixerPlan checks the arguments once; forward() on new data written into its buffers equals
    # gdn_mixer_fwd (or gdn_mixer_fwd_gates) on the same data, bit for bit, call after call.
    T, Hk, Hv = gi.MIXER_T, 16, 32
    say(f"[mixer-plan] {form} T={T}")
    m = gi.make_mixer_inputs(120)
    t = dict(qkv=bf16_dev(m.qkv), conv_w=bf16_dev(m.conv_w), g=f32_dev(m.g), beta=f32_dev(m.beta), z=bf16_dev(m.z),
             norm_w=bf16_dev(m.norm_w), cu=torch.from_numpy(m.cu.astype(np.int32)).cuda())
    cu_h = torch.from_numpy(m.cu.astype(np.int64))
    gates = None
    if form == "gates":
        gt = gi.make_gate_inputs(121, T, Hv)
        gates = (bf16_dev(gt.a), bf16_dev(gt.b), f32_dev(gt.A_log), f32_dev(gt.dt_bias))
    plan = gdn.MixerPlan(t["qkv"], t["conv_w"], None if gates else t["g"], None if gates else t["beta"], t["z"],
                         t["norm_w"], t["cu"], None, Hk=Hk, Hv=Hv, cu_seqlens_host=cu_h, gates=gates)
    for rep in range(3):
        m2 = gi.make_mixer_inputs(130 + rep)
        t["qkv"].copy_(bf16_dev(m2.qkv))
        t["z"].copy_(bf16_dev(m2.z))
        y_p, h_p = plan.forward()
        if gates:
            y_e, h_e = gdn.gdn_mixer_fwd_gates(t["qkv"], t["conv_w"], *gates, t["z"], t["norm_w"], t["cu"], None,
                                               Hk=Hk, Hv=Hv, cu_seqlens_host=cu_h)
        else:
            y_e, h_e = gdn.gdn_mixer_fwd(t["qkv"], t["conv_w"], t["g"], t["beta"], t["z"], t["norm_w"], t["cu"], None,
                                         Hk=Hk, Hv=Hv, cu_seqlens_host=cu_h)
        torch.cuda.synchronize()
        assert torch.equal(y_p.view(torch.int16), y_e.view(torch.int16)), f"call {rep}: y differs"
        assert torch.equal(h_p, h_e), f"call {rep}: hT differs"
    say("  3 plan calls bitwise equal to the function")


def test_mixer_side_stream_with_binding_allocations():
    # The binding allocates y, hT and the workspace itself; the calls run on a side stream while the
    # current stream keeps allocating and writing memory of the same sizes.  The allocations are
    # recorded on the side stream, so none of that memory may be reused under the calls.  Also
    # want_state=False: no state returned, the same y.
    T, Hk, Hv = gi.MIXER_T, 16, 32
    say(f"[mixer-side-stream] T={T} on a side stream, allocations on the current stream")
    m = gi.make_mixer_inputs(140)
    args = (bf16_dev(m.qkv), bf16_dev(m.conv_w), f32_dev(m.g), f32_dev(m.beta), bf16_dev(m.z), bf16_dev(m.norm_w),
            torch.from_numpy(m.cu.astype(np.int32)).cuda(), None)
    cu_h = torch.from_numpy(m.cu.astype(np.int64))
    y_ref, h_ref = gdn.gdn_mixer_fwd(*args, Hk=Hk, Hv=Hv, cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    ws_n = gdn.gdn_mixer_fwd_workspace_size(T, 1, Hk, Hv)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(gdn.gdn_mixer_fwd(*args, Hk=Hk, Hv=Hv, stream=side, cu_seqlens_host=cu_h))
        junk = [torch.full((ws_n,), 0xFF, dtype=torch.uint8, device="cuda"),
                torch.full((T, Hv, 128), float("nan"), dtype=torch.bfloat16, device="cuda"),
                torch.full((1, Hv, 128, 128), float("nan"), dtype=torch.float32, device="cuda")]
        del junk
    torch.cuda.current_stream().wait_stream(side)
    y_ns, h_ns = gdn.gdn_mixer_fwd(*args, Hk=Hk, Hv=Hv, want_state=False, cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    for y, hT in outs:
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)) and torch.equal(hT, h_ref)
    assert h_ns is None and torch.equal(y_ns.view(torch.int16), y_ref.view(torch.int16))
    say("  3 side-stream calls and a call without state bitwise equal to the current-stream call")
