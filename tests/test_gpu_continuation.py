"""Continuation entry points on the GPU, through the C ABI, against the fp64 oracle:

* gdn_chunk_fwd_indexed -- initial states drawn from a pool by index (one prefix state handed to
  many candidates), same tolerance as gdn_chunk_fwd, plus bitwise equality with explicit copies;
* gdn_mixer_fwd_cont -- the mixer carrying its conv input window beside the recurrent state; the
  window out is bit-exact (copied bf16 values), y and hT to the mixer tolerance, and a split at a
  chunk boundary continued from its own state and window equals one run bitwise;
* gdn_mixer_fwd_gates_cont -- the same with the gate parameters made in the first kernel."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_deltanet_chunked_amd as gdn
import gdn_inputs as gi
import oracle
from tests.gpu_util import bf16_dev, check, dev_inputs, f32_dev, say
from tests.test_gpu_mixer import check_mixer

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()


def _np(t):
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy().astype(np.float64)


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def run_indexed(x, pool, index, **kw):
    d = dev_inputs(x)
    o, hT = gdn.gdn_chunk_fwd_indexed(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], f32_dev(pool), _i32(index),
                                      cu_seqlens_host=torch.from_numpy(x.cu.astype(np.int64)), **kw)
    torch.cuda.synchronize()
    return o, hT


@pytest.mark.parametrize("Hk,Hv,lengths,S,index", [
    (16, 32, [61, 73, 88, 95, 104, 117, 139], 1, [0] * 7),          # 7 candidates of one 677-token prefix
    (2, 4, [1, 64, 0, 130, 65, 3], 3, [2, 0, 2, -1, 1, 3]),          # repeats, empty, out of range
])
def test_indexed_parity(Hk, Hv, lengths, S, index):
    say(f"[indexed] Hk={Hk} Hv={Hv} lengths={lengths} pool={S} index={index}")
    x = gi.make_gdn_inputs(Hk, Hv, lengths, seed=200 + S)
    pool = gi.make_state_pool(210 + S, S, Hv)
    o, hT = run_indexed(x, pool, index)
    q, k, v, g, b, cu, _ = x.f64()
    o_ref, h_ref = oracle.gdn_fwd_indexed(q, k, v, g, b, cu, pool.astype(np.float64), index)
    check(_np(o), _np(hT), o_ref, h_ref, "indexed")


def test_indexed_equals_copies_bitwise():
    lengths = [100, 37, 0, 64, 5]
    index = [1, 1, 0, 7, 1]
    say(f"[indexed-bitwise] lengths={lengths} index={index}")
    x = gi.make_gdn_inputs(2, 4, lengths, seed=220)
    pool = gi.make_state_pool(221, 2, 4)
    o, hT = run_indexed(x, pool, index)
    gathered = np.stack([pool[i] if 0 <= i < 2 else np.zeros_like(pool[0]) for i in index])
    d = dev_inputs(x)
    o2, h2 = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], f32_dev(gathered))
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(hT, h2)
    # identity map over a pool of N states is gdn_chunk_fwd itself
    o3, h3 = run_indexed(x, gathered, np.arange(len(lengths)))
    assert torch.equal(o.view(torch.int16), o3.view(torch.int16)) and torch.equal(hT, h3)


def test_indexed_full_size_fanout():
    # the 539-token single-sequence workload, continued from state 1 of a pool of 4
    say("[indexed-full] t539_h16x32 from pool state 1 of 4")
    x = gi.make_case("t539_h16x32")
    pool = gi.make_state_pool(230, 4, 32)
    o, hT = run_indexed(x, pool, [1])
    q, k, v, g, b, cu, _ = x.f64()
    o_ref, h_ref = oracle.gdn_fwd_indexed(q, k, v, g, b, cu, pool.astype(np.float64), [1])
    check(_np(o), _np(hT), o_ref, h_ref, "t539 fan-out")


# ---------------------------------------------------------------------------------------------
# Mixer continuation
# ---------------------------------------------------------------------------------------------
def run_cont(m, h0, win, index, Hk, Hv, **kw):
    y, hT, wout = gdn.gdn_mixer_fwd_cont(
        bf16_dev(m.qkv), bf16_dev(m.conv_w), f32_dev(m.g), f32_dev(m.beta), bf16_dev(m.z), bf16_dev(m.norm_w),
        _i32(m.cu), None if h0 is None else (h0 if torch.is_tensor(h0) else f32_dev(h0)),
        None if win is None else (win if torch.is_tensor(win) else bf16_dev(win)),
        None if index is None else _i32(index), Hk=Hk, Hv=Hv,
        cu_seqlens_host=torch.from_numpy(m.cu.astype(np.int64)), **kw)
    torch.cuda.synchronize()
    return y, hT, wout


def cont_oracle(m, h0, win, index, Hk, Hv):
    """(y, hT, conv_out, o) from the oracle; o (the rule's output at its bf16 point) only scales the
    elementwise bound on y, and is rebuilt from the oracle's pieces with the same window and state."""
    f = gi.bits_to_f64
    h0d = None if h0 is None else h0.astype(np.float64)
    wd = None if win is None else f(win)
    y, hT, wout = oracle.mixer_fwd_cont(f(m.qkv), f(m.conv_w), m.g, m.beta, f(m.z), f(m.norm_w), m.cu, h0d, wd,
                                        index, Hk=Hk, Hv=Hv)
    T, d = m.qkv.shape[0], 128
    a, _ = oracle.conv_silu_cont(f(m.qkv), f(m.conv_w), m.cu, wd, index)
    l2 = lambda x: x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)
    q = oracle.round_bf16(l2(a[:, :Hk * d].reshape(T, Hk, d)))
    k = oracle.round_bf16(l2(a[:, Hk * d:2 * Hk * d].reshape(T, Hk, d)))
    v = oracle.round_bf16(a[:, 2 * Hk * d:].reshape(T, Hv, d))
    N = len(m.cu) - 1
    pool = h0d if h0d is not None else np.zeros((1, Hv, d, d))
    idx = index if index is not None else np.arange(N)
    if h0d is None:
        idx = np.full(N, -1)
    o, _ = oracle.gdn_fwd_indexed(q, k, v, m.g, m.beta, m.cu, pool, idx)
    return y, hT, wout, oracle.round_bf16(o)


@pytest.mark.parametrize("Hk,Hv,lengths,S,index", [
    (2, 4, [1, 2, 0, 70, 3, 130], 3, [2, 0, 1, 1, -1, 2]),
    (16, 32, [61, 73, 88, 95, 104, 117, 139], 1, [0] * 7),
])
def test_mixer_cont_parity(Hk, Hv, lengths, S, index):
    say(f"[mixer-cont] Hk={Hk} Hv={Hv} lengths={lengths} pool={S} index={index}")
    m = gi.make_mixer_inputs(240 + S, lengths=lengths, Hk=Hk, Hv=Hv)
    C = m.qkv.shape[1]
    h0 = gi.make_state_pool(250 + S, S, Hv)
    win = gi.make_window_pool(260 + S, S, C)
    y, hT, wout = run_cont(m, h0, win, index, Hk, Hv)
    y_ref, h_ref, w_ref, o_ref = cont_oracle(m, h0, win, index, Hk, Hv)
    assert np.array_equal(_np(wout), w_ref), "conv window out (bit-exact)"
    check_mixer(_np(y), _np(hT), y_ref, h_ref, o_ref, "mixer cont", m)


@pytest.mark.parametrize("split", [64, 128, 37])
def test_mixer_cont_split(split):
    lengths = [300, 200]
    say(f"[mixer-split] lengths={lengths} split={split}")
    m = gi.make_mixer_inputs(270, lengths=lengths, Hk=2, Hv=4, with_h0=True)
    y, hT, wout = run_cont(m, m.h0, None, None, 2, 4)
    cu = m.cu
    head = np.concatenate([np.arange(cu[n], cu[n] + split) for n in range(2)])
    tail = np.concatenate([np.arange(cu[n] + split, cu[n + 1]) for n in range(2)])
    part = lambda rows, cu2: gi.MixerInputs(m.qkv[rows], m.conv_w, m.beta[rows], m.g[rows], m.z[rows], m.norm_w,
                                            np.asarray(cu2, np.int32))
    ya, ha, wa = run_cont(part(head, [0, split, 2 * split]), m.h0, None, None, 2, 4)
    mb = part(tail, [0, 300 - split, 500 - 2 * split])
    yb, hb, wb = run_cont(mb, ha, wa, None, 2, 4)
    yy = torch.empty_like(y)
    yy[torch.from_numpy(head).cuda()] = ya
    yy[torch.from_numpy(tail).cuda()] = yb
    assert torch.equal(wb.view(torch.int16), wout.view(torch.int16)), "window out after continuation"
    if split % 64 == 0:
        assert torch.equal(yy.view(torch.int16), y.view(torch.int16)) and torch.equal(hb, hT), \
            "a split at a chunk boundary continues bitwise"
    y_ref, h_ref, w_ref, o_ref = cont_oracle(m, m.h0, None, None, 2, 4)
    check_mixer(_np(yy), _np(hb), y_ref, h_ref, o_ref, f"split {split}", m)


def test_mixer_cont_in_place_and_plain_entry():
    lengths = [50, 2, 77]
    say(f"[mixer-inplace] lengths={lengths}")
    m = gi.make_mixer_inputs(280, lengths=lengths, Hk=2, Hv=4)
    C = m.qkv.shape[1]
    h0 = gi.make_state_pool(281, 3, 4)
    win = gi.make_window_pool(282, 3, C)
    y1, h1, w1 = run_cont(m, h0, win, None, 2, 4)
    hbuf, wbuf = f32_dev(h0), bf16_dev(win)
    y2, h2, w2 = run_cont(m, hbuf, wbuf, None, 2, 4, hT=hbuf, conv_out=wbuf)
    assert h2.data_ptr() == hbuf.data_ptr() and w2.data_ptr() == wbuf.data_ptr()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)) and torch.equal(h1, h2)
    assert torch.equal(w1.view(torch.int16), w2.view(torch.int16))
    # gdn_mixer_fwd is the continued form with no window and no index
    y3, h3 = gdn.gdn_mixer_fwd(bf16_dev(m.qkv), bf16_dev(m.conv_w), f32_dev(m.g), f32_dev(m.beta), bf16_dev(m.z),
                               bf16_dev(m.norm_w), _i32(m.cu), f32_dev(h0), Hk=2, Hv=4)
    y4, h4, _ = run_cont(m, h0, None, None, 2, 4)
    torch.cuda.synchronize()
    assert torch.equal(y3.view(torch.int16), y4.view(torch.int16)) and torch.equal(h3, h4)


def test_mixer_gates_cont_split():
    # The gates made from the projections, continued across a split at a chunk boundary from the
    # first part's state and window, equal one gdn_mixer_fwd_gates run bit for bit; a pooled,
    # indexed continuation against the oracle fed the oracle's gates.
    lengths = [300, 200]
    split = 128
    say(f"[mixer-gates-cont] lengths={lengths} split={split}")
    m = gi.make_mixer_inputs(290, lengths=lengths, Hk=2, Hv=4, with_h0=True)
    gt = gi.make_gate_inputs(291, m.qkv.shape[0], 4)
    dev = lambda rows=None: (bf16_dev(gt.a if rows is None else gt.a[rows]), bf16_dev(gt.b if rows is None else gt.b[rows]),
                             f32_dev(gt.A_log), f32_dev(gt.dt_bias))
    y, hT = gdn.gdn_mixer_fwd_gates(bf16_dev(m.qkv), bf16_dev(m.conv_w), *dev(), bf16_dev(m.z), bf16_dev(m.norm_w),
                                    _i32(m.cu), f32_dev(m.h0), Hk=2, Hv=4,
                                    cu_seqlens_host=torch.from_numpy(m.cu.astype(np.int64)))
    cu = m.cu
    head = np.concatenate([np.arange(cu[n], cu[n] + split) for n in range(2)])
    tail = np.concatenate([np.arange(cu[n] + split, cu[n + 1]) for n in range(2)])

    def part(rows, cu2, h0, win):
        c2 = np.asarray(cu2, np.int32)
        return gdn.gdn_mixer_fwd_gates_cont(bf16_dev(m.qkv[rows]), bf16_dev(m.conv_w), *dev(rows),
                                            bf16_dev(m.z[rows]), bf16_dev(m.norm_w), _i32(c2), h0, win, None,
                                            Hk=2, Hv=4, cu_seqlens_host=torch.from_numpy(c2.astype(np.int64)))

    ya, ha, wa = part(head, [0, split, 2 * split], f32_dev(m.h0), None)
    yb, hb, wb = part(tail, [0, 300 - split, 500 - 2 * split], ha, wa)
    torch.cuda.synchronize()
    yy = torch.empty_like(y)
    yy[torch.from_numpy(head).cuda()] = ya
    yy[torch.from_numpy(tail).cuda()] = yb
    assert torch.equal(yy.view(torch.int16), y.view(torch.int16)) and torch.equal(hb, hT), \
        "a split at a chunk boundary continues bitwise"
    # pooled states and windows by index, against the oracle with its own gates
    S, index = 3, np.array([2, -1], np.int32)
    C = m.qkv.shape[1]
    h0p, winp = gi.make_state_pool(292, S, 4), gi.make_window_pool(293, S, C)
    yc, hc, wc = gdn.gdn_mixer_fwd_gates_cont(bf16_dev(m.qkv), bf16_dev(m.conv_w), *dev(), bf16_dev(m.z),
                                              bf16_dev(m.norm_w), _i32(m.cu), f32_dev(h0p), bf16_dev(winp),
                                              _i32(index), Hk=2, Hv=4,
                                              cu_seqlens_host=torch.from_numpy(m.cu.astype(np.int64)))
    torch.cuda.synchronize()
    f = gi.bits_to_f64
    g, beta = oracle.gates(f(gt.a), f(gt.b), gt.A_log.astype(np.float64), gt.dt_bias.astype(np.float64))
    mg = dataclasses.replace(m, g=g, beta=beta)
    y_ref, h_ref, w_ref, o_ref = cont_oracle(mg, h0p, winp, index, 2, 4)
    assert np.array_equal(_np(wc), w_ref), "conv window out (bit-exact)"
    check_mixer(_np(yc), _np(hc), y_ref, h_ref, o_ref, "gates cont (indexed)", mg)
