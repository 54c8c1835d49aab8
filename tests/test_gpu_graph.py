"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: no call
allocates when its outputs and workspace are given, and no kernel uses a memset, so a serving loop
can capture a layer's launches once.  Each test writes new inputs into the captured buffers,
replays, and compares every replay bitwise with an eager call on the same inputs, with eager work
and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_amd as gdn
import gdn_inputs as gi
from tests.gpu_util import bf16_dev, check, dev_inputs, f32_dev, run_oracle, say

pytestmark = pytest.mark.gpu

_KEYS = ("q", "k", "v", "g", "beta", "h0")


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("tag,Hk,Hv,lengths,with_h0", [
    ("single round T=539", 16, 32, [539], False),
    ("time split T=3000", 2, 4, [3000], True),
    ("persistent 7 sequences", 16, 32, [61, 73, 88, 95, 104, 117, 139], True),
])
def test_graph_replay_chunk_fwd(tag, Hk, Hv, lengths, with_h0):
    say(f"[graph] gdn_chunk_fwd {tag}")
    xs = [gi.make_gdn_inputs(Hk, Hv, lengths, seed=700 + s, with_h0=with_h0) for s in range(3)]
    d = dev_inputs(xs[0])
    cu_h = torch.from_numpy(xs[0].cu.astype(np.int64))
    T, N = int(xs[0].cu[-1]), len(lengths)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(T, N, Hk, Hv), dtype=torch.uint8, device="cuda")
    plan = gdn.ChunkPlan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], d["h0"], workspace=ws,
                         cu_seqlens_host=cu_h)
    graph = _capture(plan.forward)
    for i, x in enumerate(xs):
        new = dev_inputs(x)
        for key in _KEYS:
            if d[key] is not None:
                d[key].copy_(new[key])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_g, h_g = plan.o.clone(), plan.hT.clone()
        o_e, h_e = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], d["h0"],
                                     cu_seqlens_host=cu_h)
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), f"replay {i}: o differs from eager"
        assert torch.equal(h_g, h_e), f"replay {i}: hT differs from eager"
        if i == 0:
            check(o_g.float().cpu().numpy().astype(np.float64), h_g.cpu().numpy().astype(np.float64),
                  *run_oracle(x), f"{tag} replay 0")
    say(f"  {len(xs)} replays bitwise equal to eager calls")


def test_graph_replay_mixer_layers():
    # two mixer layers (input prep + chunk prep, state pass, gated RMSNorm each) in one graph
    T, Hk, Hv, D = gi.MIXER_T, 16, 32, 128
    say(f"[graph] two gdn_mixer_fwd layers T={T}")
    layers = []
    for l in range(2):
        m = gi.make_mixer_inputs(800 + l)
        layers.append(dict(qkv=bf16_dev(m.qkv), conv_w=bf16_dev(m.conv_w), g=f32_dev(m.g), beta=f32_dev(m.beta),
                           z=bf16_dev(m.z), norm_w=bf16_dev(m.norm_w), cu=torch.from_numpy(m.cu.astype(np.int32)).cuda(),
                           y=torch.empty((T, Hv, D), dtype=torch.bfloat16, device="cuda"),
                           hT=torch.empty((1, Hv, D, D), dtype=torch.float32, device="cuda")))
    cu_h = torch.tensor([0, T], dtype=torch.int64)
    ws = torch.empty(gdn.gdn_mixer_fwd_workspace_size(T, 1, Hk, Hv), dtype=torch.uint8, device="cuda")

    def run(outs=None):
        res = []
        for L in layers:
            y, hT = gdn.gdn_mixer_fwd(L["qkv"], L["conv_w"], L["g"], L["beta"], L["z"], L["norm_w"], L["cu"], None,
                                      Hk=Hk, Hv=Hv, y=None if outs == "fresh" else L["y"],
                                      hT=None if outs == "fresh" else L["hT"], workspace=ws, cu_seqlens_host=cu_h)
            res.append((y, hT))
        return res

    graph = _capture(run)
    for rep in range(3):
        for l, L in enumerate(layers):
            m = gi.make_mixer_inputs(900 + 10 * rep + l)
            L["qkv"].copy_(bf16_dev(m.qkv))
            L["z"].copy_(bf16_dev(m.z))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [(L["y"].clone(), L["hT"].clone()) for L in layers]
        eager = run("fresh")
        torch.cuda.synchronize()
        for l, ((y_g, h_g), (y_e, h_e)) in enumerate(zip(got, eager)):
            assert torch.equal(y_g.view(torch.int16), y_e.view(torch.int16)), f"replay {rep} layer {l}: y differs"
            assert torch.equal(h_g, h_e), f"replay {rep} layer {l}: hT differs"
    say("  3 replays of two layers bitwise equal to eager calls")


def test_graph_replay_mixer_plan_gates():
    # a MixerPlan with the gates made in the first kernel and an initial state, captured once
    T, Hk, Hv = gi.MIXER_T, 16, 32
    say(f"[graph] MixerPlan with gates and h0, T={T}")
    m = gi.make_mixer_inputs(820, with_h0=True)
    gt = gi.make_gate_inputs(821, T, Hv)
    t = dict(qkv=bf16_dev(m.qkv), conv_w=bf16_dev(m.conv_w), z=bf16_dev(m.z), norm_w=bf16_dev(m.norm_w),
             cu=torch.from_numpy(m.cu.astype(np.int32)).cuda(), h0=f32_dev(m.h0))
    gates = (bf16_dev(gt.a), bf16_dev(gt.b), f32_dev(gt.A_log), f32_dev(gt.dt_bias))
    cu_h = torch.from_numpy(m.cu.astype(np.int64))
    plan = gdn.MixerPlan(t["qkv"], t["conv_w"], None, None, t["z"], t["norm_w"], t["cu"], t["h0"], Hk=Hk, Hv=Hv,
                         cu_seqlens_host=cu_h, gates=gates)
    graph = _capture(plan.forward)
    for rep in range(3):
        m2 = gi.make_mixer_inputs(830 + rep, with_h0=True)
        g2 = gi.make_gate_inputs(840 + rep, T, Hv)
        t["qkv"].copy_(bf16_dev(m2.qkv))
        t["z"].copy_(bf16_dev(m2.z))
        t["h0"].copy_(f32_dev(m2.h0))
        gates[0].copy_(bf16_dev(g2.a))
        gates[1].copy_(bf16_dev(g2.b))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y_g, h_g = plan.y.clone(), plan.hT.clone()
        y_e, h_e = gdn.gdn_mixer_fwd_gates(t["qkv"], t["conv_w"], *gates, t["z"], t["norm_w"], t["cu"], t["h0"],
                                           Hk=Hk, Hv=Hv, cu_seqlens_host=cu_h)
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), y_e.view(torch.int16)), f"replay {rep}: y differs"
        assert torch.equal(h_g, h_e), f"replay {rep}: hT differs"
    say("  3 replays bitwise equal to eager calls")


def test_graph_replay_mixer_cont_in_place():
    # A prefill taken piece by piece from a captured graph: one gdn_mixer_fwd_cont call whose state
    # and conv window pools are updated in place (hT = h0, conv_out = conv_in), so every replay
    # continues from the previous one.  Each replay equals the same call made eagerly on pools that
    # went through the same pieces.
    Hk, Hv, D, lengths = 2, 4, 128, [64, 37]
    say(f"[graph] gdn_mixer_fwd_cont in place, pieces of lengths {lengths}")
    m = gi.make_mixer_inputs(850, lengths=lengths, Hk=Hk, Hv=Hv)
    C, T = m.qkv.shape[1], int(m.cu[-1])
    t = dict(qkv=bf16_dev(m.qkv), conv_w=bf16_dev(m.conv_w), g=f32_dev(m.g), beta=f32_dev(m.beta), z=bf16_dev(m.z),
             norm_w=bf16_dev(m.norm_w), cu=torch.from_numpy(m.cu.astype(np.int32)).cuda())
    cu_h = torch.from_numpy(m.cu.astype(np.int64))
    h_pool, w_pool = f32_dev(gi.make_state_pool(851, 2, Hv)), bf16_dev(gi.make_window_pool(852, 2, C))
    h_eager, w_eager = h_pool.clone(), w_pool.clone()
    y = torch.empty((T, Hv, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.gdn_mixer_fwd_workspace_size(T, 2, Hk, Hv), dtype=torch.uint8, device="cuda")

    def call(h, w, out):
        return gdn.gdn_mixer_fwd_cont(t["qkv"], t["conv_w"], t["g"], t["beta"], t["z"], t["norm_w"], t["cu"], h, w,
                                      Hk=Hk, Hv=Hv, y=out, hT=h, conv_out=w, workspace=ws, cu_seqlens_host=cu_h)

    h_start, w_start = h_pool.clone(), w_pool.clone()
    graph = _capture(lambda: call(h_pool, w_pool, y))
    h_pool.copy_(h_start)  # the warm-up and the capture may have advanced the pools
    w_pool.copy_(w_start)
    for rep in range(4):
        p = gi.make_mixer_inputs(860 + rep, lengths=lengths, Hk=Hk, Hv=Hv)
        for key, val in (("qkv", bf16_dev(p.qkv)), ("g", f32_dev(p.g)), ("beta", f32_dev(p.beta)), ("z", bf16_dev(p.z))):
            t[key].copy_(val)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y_g = y.clone()
        y_e, _, _ = call(h_eager, w_eager, None)
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), y_e.view(torch.int16)), f"piece {rep}: y differs"
        assert torch.equal(h_pool, h_eager), f"piece {rep}: state pool differs"
        assert torch.equal(w_pool.view(torch.int16), w_eager.view(torch.int16)), f"piece {rep}: window pool differs"
    say("  4 pieces replayed, each bitwise equal to the eager continuation")
