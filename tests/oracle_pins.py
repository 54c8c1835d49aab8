"""Pins for the fp64 oracle: facts fixed by the mathematics, not by the oracle itself.

Each ``pin_*`` takes ``fwd`` -- a callable with the signature of ``oracle.gdn_fwd`` -- and
raises ``AssertionError`` when the implementation behind it disagrees with a closed form, an
identity, an exact rational result or an invariant of the gated delta rule

    S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t

(Gated DeltaNet, cited by the "open-jev-fast" README, "Phase 3" item 1, reference [5]).
State arrays h0 / hT are key-major [N, Hv, dk, dv] (H = S^T).

The same pins run against the real oracle (test_oracle_pins.py) and against deliberately
broken copies of it (test_oracle_mutants.py), which shows that each plausible mistake is
caught by at least one pin.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _rel(a, b):
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def _rand_case(rng, T, Hk, Hv, d, lengths=None, h0=True, gmean=1.0):
    lengths = lengths or [T]
    T = sum(lengths)
    q = rng.standard_normal((T, Hk, d)) / np.sqrt(d)
    k = rng.standard_normal((T, Hk, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, d))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))
    g = -np.log1p(np.exp(-(gmean + rng.standard_normal((T, Hv)))))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    H0 = rng.standard_normal((len(lengths), Hv, d, d)) * 0.3 if h0 else None
    return q, k, v, g, beta, cu, H0


# ------------------------------------------------------------------------------------------
# P-1: beta = 0  =>  S_t = e^{G_t} S_0 and o_t = e^{G_t} S_0 q_t  (needs a non-zero, non-symmetric h0)
# ------------------------------------------------------------------------------------------
def pin_beta_zero_decay(fwd):
    rng = np.random.default_rng(11)
    q, k, v, g, beta, cu, h0 = _rand_case(rng, 0, 2, 4, 8, lengths=[9, 5])
    beta[:] = 0.0
    o, hT = fwd(q, k, v, g, beta, cu, h0)
    for n in range(2):
        for h in range(4):
            S0 = h0[n, h].T  # value-major
            G = 0.0
            for t in range(cu[n], cu[n + 1]):
                G += g[t, h]
                exp_o = np.exp(G) * S0 @ q[t, h // 2]
                assert np.allclose(o[t, h], exp_o, rtol=1e-12, atol=1e-13), "beta=0 output"
            assert np.allclose(hT[n, h], np.exp(G) * h0[n, h], rtol=1e-12, atol=1e-13), "beta=0 state"


# ------------------------------------------------------------------------------------------
# P-2: g = 0, beta = 1, orthonormal keys, S_0 = 0  =>  exact key -> value retrieval
# ------------------------------------------------------------------------------------------
def pin_orthonormal_retrieval(fwd, d=16, T=12, Hk=1, Hv=2):
    rng = np.random.default_rng(12)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm[:T]  # T orthonormal rows
    k = np.repeat(keys[:, None, :], Hk, axis=1)
    v = rng.standard_normal((T, Hv, d))
    src = np.array([rng.integers(0, t + 1) for t in range(T)])  # query t retrieves key src[t] <= t
    q = np.repeat(keys[src][:, None, :], Hk, axis=1)
    g = np.zeros((T, Hv))
    beta = np.ones((T, Hv))
    o, hT = fwd(q, k, v, g, beta, [0, T], None)
    for t in range(T):
        for h in range(Hv):
            assert np.allclose(o[t, h], v[src[t], h], atol=1e-12), "retrieval"
    for h in range(Hv):
        S = sum(np.outer(v[t, h], keys[t]) for t in range(T))
        assert np.allclose(hT[0, h], S.T, atol=1e-12), "retrieval state"


# ------------------------------------------------------------------------------------------
# P-3: the chunked (WY / UT-transform) form equals the recurrence in fp64.
# Written from the algebra: with H = S^T, local cumsum G inside a chunk,
#   A_ij = beta_i e^{G_i-G_j} k_i.k_j (i>j), T = (I+A)^{-1},
#   W = T diag(beta e^G) K, U = T diag(beta) V, U~ = U - W H,
#   O = diag(e^G) Q H + (M o Q K^T) U~,  M_ij = e^{G_i-G_j} (i>=j),
#   H' = e^{G_C} H + K^T diag(e^{G_C - G}) U~.
# ------------------------------------------------------------------------------------------
def chunked_reference(q, k, v, g, beta, cu, h0, C=64):
    T, Hk, d = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    N = len(cu) - 1
    o = np.zeros((T, Hv, dv))
    hT = np.zeros((N, Hv, d, dv))
    for n in range(N):
        for h in range(Hv):
            hk = h // (Hv // Hk)
            H = h0[n, h].copy() if h0 is not None else np.zeros((d, dv))
            for c0 in range(cu[n], cu[n + 1], C):
                sl = slice(c0, min(c0 + C, cu[n + 1]))
                K, Q, V = k[sl, hk], q[sl, hk], v[sl, h]
                b = beta[sl, h]
                G = np.cumsum(g[sl, h])
                L = len(G)
                Dm = np.exp(G[:, None] - np.where(np.tril(np.ones((L, L))) > 0, G[None, :], np.inf))
                A = np.tril(b[:, None] * Dm * (K @ K.T), -1)
                Tm = np.linalg.inv(np.eye(L) + A)
                W = Tm @ (b[:, None] * np.exp(G)[:, None] * K)
                U = Tm @ (b[:, None] * V)
                Ut = U - W @ H
                o[sl, h] = np.exp(G)[:, None] * (Q @ H) + (Dm * (Q @ K.T)) @ Ut
                H = np.exp(G[-1]) * H + K.T @ (np.exp(G[-1] - G)[:, None] * Ut)
            hT[n, h] = H
    return o, hT


def pin_chunked_identity(fwd):
    rng = np.random.default_rng(13)
    # several chunks, ragged tails, empty sequence, GQA, non-zero initial states
    q, k, v, g, beta, cu, h0 = _rand_case(rng, 0, 2, 4, 16, lengths=[150, 0, 64, 1, 65, 129], gmean=3.0)
    o, hT = fwd(q, k, v, g, beta, cu, h0)
    oc, hc = chunked_reference(q, k, v, g, beta, cu, h0)
    assert _rel(o, oc) < 1e-12, f"chunked identity (o) {_rel(o, oc)}"
    assert _rel(hT, hc) < 1e-12, f"chunked identity (hT) {_rel(hT, hc)}"


# ------------------------------------------------------------------------------------------
# P-4: a packed batch equals separate runs (bitwise in the oracle)
# ------------------------------------------------------------------------------------------
def pin_varlen_equals_separate(fwd):
    rng = np.random.default_rng(14)
    lengths = [7, 0, 30, 3]
    q, k, v, g, beta, cu, h0 = _rand_case(rng, 0, 2, 4, 8, lengths=lengths)
    o, hT = fwd(q, k, v, g, beta, cu, h0)
    for n, L in enumerate(lengths):
        sl = slice(cu[n], cu[n + 1])
        o1, h1 = fwd(q[sl], k[sl], v[sl], g[sl], beta[sl], [0, L], h0[n:n + 1])
        assert np.array_equal(o[sl], o1), "varlen output"
        assert np.array_equal(hT[n], h1[0]), "varlen state"


# ------------------------------------------------------------------------------------------
# P-5: exact rational brute force (sum-of-products closed form) -- stored worked example
#      written by tests/golden/make_golden.py, and a fresh random one
# ------------------------------------------------------------------------------------------
def _frac(s):
    return Fraction(s)


def pin_golden_exact(fwd):
    with open(os.path.join(HERE, "golden", "brute_d4_t6.json")) as f:
        doc = json.load(f)
    alpha = np.array([float(_frac(x)) for x in doc["alpha"]])
    beta = np.array([float(_frac(x)) for x in doc["beta"]])[:, None]
    q = np.array([[float(_frac(x)) for x in r] for r in doc["q"]])[:, None, :]
    k = np.array([[float(_frac(x)) for x in r] for r in doc["k"]])[:, None, :]
    v = np.array([[float(_frac(x)) for x in r] for r in doc["v"]])[:, None, :]
    S0 = np.array([[float(_frac(x)) for x in r] for r in doc["S0_value_major"]])
    o_ex = np.array([[float(_frac(x)) for x in r] for r in doc["o"]])
    S_ex = np.array([[float(_frac(x)) for x in r] for r in doc["ST_value_major"]])
    g = np.log(alpha)[:, None]
    o, hT = fwd(q, k, v, g, beta, [0, len(alpha)], S0.T[None, None])
    assert np.allclose(o[:, 0, :], o_ex, rtol=1e-13, atol=1e-14), "golden o"
    assert np.allclose(hT[0, 0], S_ex.T, rtol=1e-13, atol=1e-14), "golden hT"


def pin_brute_random(fwd, T=5, d=3, seed=15):
    from oracle import brute
    rng = np.random.default_rng(seed)
    R = lambda: Fraction(int(rng.integers(-8, 9)), 8)
    alpha = [Fraction(int(rng.integers(1, 9)), 8) for _ in range(T)]
    beta = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    q = [[R() for _ in range(d)] for _ in range(T)]
    k = [[R() for _ in range(d)] for _ in range(T)]
    v = [[R() for _ in range(d)] for _ in range(T)]
    S0 = [[R() for _ in range(d)] for _ in range(d)]
    outs, ST = brute.run(alpha, beta, q, k, v, S0)
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    o, hT = fwd(f(q)[:, None], f(k)[:, None], f(v)[:, None], np.log(np.array([float(a) for a in alpha]))[:, None],
                np.array([float(b) for b in beta])[:, None], [0, T], f(S0).T[None, None])
    assert np.allclose(o[:, 0], f(outs), rtol=1e-12, atol=1e-13), "brute o"
    assert np.allclose(hT[0, 0], f(ST).T, rtol=1e-12, atol=1e-13), "brute hT"


# ------------------------------------------------------------------------------------------
# P-6: continuation -- run [0, s) then [s, T) from its final state == one run (bitwise)
# ------------------------------------------------------------------------------------------
def pin_continuation(fwd):
    rng = np.random.default_rng(16)
    q, k, v, g, beta, cu, h0 = _rand_case(rng, 0, 2, 2, 8, lengths=[40])
    o, hT = fwd(q, k, v, g, beta, cu, h0)
    for s in (1, 17, 39):
        oa, ha = fwd(q[:s], k[:s], v[:s], g[:s], beta[:s], [0, s], h0)
        ob, hb = fwd(q[s:], k[s:], v[s:], g[s:], beta[s:], [0, 40 - s], ha)
        assert np.array_equal(np.concatenate([oa, ob]), o), "continuation output"
        assert np.array_equal(hb, hT), "continuation state"


# ------------------------------------------------------------------------------------------
# P-7: T = 1 closed form  o = e^g S_0 q + beta (v - e^g S_0 k)(k.q)
# ------------------------------------------------------------------------------------------
def pin_first_token(fwd):
    rng = np.random.default_rng(17)
    d = 6
    q, k, v, g, beta, cu, h0 = _rand_case(rng, 0, 1, 1, d, lengths=[1])
    o, hT = fwd(q, k, v, g, beta, cu, h0)
    S0 = h0[0, 0].T
    a = np.exp(g[0, 0])
    u = beta[0, 0] * (v[0, 0] - a * S0 @ k[0, 0])
    assert np.allclose(o[0, 0], a * S0 @ q[0, 0] + u * (k[0, 0] @ q[0, 0]), rtol=1e-13, atol=1e-14), "T=1 o"
    assert np.allclose(hT[0, 0], (a * S0 + np.outer(u, k[0, 0])).T, rtol=1e-13, atol=1e-14), "T=1 hT"


# ------------------------------------------------------------------------------------------
# P-8: one repeated unit key, beta = 1, g = 0  =>  S_t k = v_t (last write wins)
# ------------------------------------------------------------------------------------------
def pin_last_write_wins(fwd):
    rng = np.random.default_rng(18)
    d, T = 8, 6
    key = rng.standard_normal(d)
    key /= np.linalg.norm(key)
    k = np.tile(key, (T, 1, 1))
    q = k.copy()
    v = rng.standard_normal((T, 1, d))
    h0 = rng.standard_normal((1, 1, d, d))
    o, _ = fwd(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), [0, T], h0)
    assert np.allclose(o[:, 0], v[:, 0], atol=1e-12), "last write wins"


# ------------------------------------------------------------------------------------------
# P-9: grouped heads -- Hk < Hv equals Hk = Hv with q/k heads duplicated (v-head h -> h // (Hv/Hk))
# ------------------------------------------------------------------------------------------
def pin_gqa_duplicated(fwd):
    rng = np.random.default_rng(19)
    q, k, v, g, beta, cu, h0 = _rand_case(rng, 0, 2, 6, 8, lengths=[20])
    o, hT = fwd(q, k, v, g, beta, cu, h0)
    idx = np.arange(6) // 3
    o2, h2 = fwd(q[:, idx], k[:, idx], v, g, beta, cu, h0)
    assert np.array_equal(o, o2) and np.array_equal(hT, h2), "GQA head map"


ALL_PINS = [pin_beta_zero_decay, pin_orthonormal_retrieval, pin_chunked_identity, pin_varlen_equals_separate,
            pin_golden_exact, pin_brute_random, pin_continuation, pin_first_token, pin_last_write_wins,
            pin_gqa_duplicated]


# ------------------------------------------------------------------------------------------
# P-9 (mixer): conv against torch's depthwise conv1d, delta taps, and the whole mixer against
# torch library pieces (conv1d, silu, rms_norm) around the pinned recurrence.  All fp64, CPU.
# Each takes (conv, mixer, fwd) with the signatures of oracle.conv_silu / mixer_fwd / gdn_fwd.
# ------------------------------------------------------------------------------------------
def _torch_conv_silu(x, w, cu):
    import torch
    import torch.nn.functional as F
    taps = w.shape[1]
    out = np.zeros_like(x)
    for n in range(len(cu) - 1):
        if cu[n + 1] == cu[n]:
            continue
        seg = torch.from_numpy(x[cu[n]:cu[n + 1]].T.copy())[None]  # [1, C, L]
        seg = F.pad(seg, (taps - 1, 0))
        y = F.conv1d(seg, torch.from_numpy(w.copy())[:, None, :], groups=x.shape[1])
        out[cu[n]:cu[n + 1]] = F.silu(y)[0].T.numpy()
    return out


def pin_conv_torch(conv, mixer, fwd):
    rng = np.random.default_rng(31)
    x = rng.standard_normal((40, 24))
    w = 0.5 * rng.standard_normal((24, 4))
    cu = [0, 3, 3, 21, 40]
    assert np.allclose(conv(x, w, cu), _torch_conv_silu(x, w, np.array(cu)), rtol=1e-12, atol=1e-13), "conv"


def pin_conv_delta_taps(conv, mixer, fwd):
    rng = np.random.default_rng(32)
    x = rng.standard_normal((10, 5))
    w = np.zeros((5, 4))
    w[:, 3] = 1.0
    assert np.allclose(conv(x, w, [0, 4, 10]), x / (1 + np.exp(-x)), rtol=1e-14), "current-token tap"
    w2 = np.zeros((5, 4))
    w2[:, 2] = 1.0  # previous token: never across a sequence start
    out = conv(x, w2, [0, 4, 10])
    assert np.all(out[[0, 4]] == 0.0) and np.allclose(out[5], x[4] / (1 + np.exp(-x[4]))), "sequence start"


def pin_mixer_torch(conv, mixer, fwd):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(33)
    Hk, Hv, d, T = 2, 4, 8, 30
    C = 2 * Hk * d + Hv * d
    cu = np.array([0, 11, 30])
    qkv = rng.standard_normal((T, C))
    cw = 0.5 * rng.standard_normal((C, 4))
    g = -np.log1p(np.exp(-(3 + rng.standard_normal((T, Hv)))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    z = rng.standard_normal((T, Hv, d))
    nw = 1 + 0.1 * rng.standard_normal(d)
    h0 = 0.1 * rng.standard_normal((2, Hv, d, d))
    a = torch.from_numpy(_torch_conv_silu(qkv, cw, cu))
    # L2 norm x / sqrt(sum x^2 + 1e-6) through the library RMSNorm: rms_norm(x, eps/d) / sqrt(d)
    l2 = lambda x: F.rms_norm(x, (d,), eps=1e-6 / d) / np.sqrt(d)
    # bf16 rounding points through torch's own fp32 -> bf16 conversion (the prepped values are
    # not ties at fp32 precision for these inputs, so fp64 -> fp32 -> bf16 is a single rounding)
    to_bf16 = lambda x: x.float().to(torch.bfloat16).double()
    for points in (False, True):
        rnd = to_bf16 if points else (lambda x: x)
        y, hT = mixer(qkv, cw, g, beta, z, nw, cu, h0, Hk=Hk, Hv=Hv, dk=d, dv=d, bf16_points=points)
        q = rnd(l2(a[:, :Hk * d].reshape(T, Hk, d)))
        k = rnd(l2(a[:, Hk * d:2 * Hk * d].reshape(T, Hk, d)))
        v = rnd(a[:, 2 * Hk * d:].reshape(T, Hv, d))
        o, hT2 = fwd(q.numpy(), k.numpy(), v.numpy(), g, beta, cu, h0)
        o = rnd(torch.from_numpy(o))
        y2 = F.rms_norm(o, (d,), torch.from_numpy(nw), eps=1e-6) * F.silu(torch.from_numpy(z))
        assert np.allclose(y, y2.numpy(), rtol=1e-11, atol=1e-12), f"mixer y (bf16 points {points})"
        assert np.allclose(hT, hT2, rtol=1e-11, atol=1e-12), f"mixer hT (bf16 points {points})"


def pin_round_bf16_matches_torch(conv, mixer, fwd, lib=None):
    import torch
    import oracle
    rng = np.random.default_rng(34)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000),
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3.0e38, -2.5e-30])])
    x32 = x.astype(np.float32).astype(np.float64)          # fp32-representable: one rounding in torch
    ref = torch.from_numpy(x32).float().to(torch.bfloat16).double().numpy()
    rnd = mixer.keywords["lib"] if hasattr(mixer, "keywords") and "lib" in mixer.keywords else None
    got = oracle.round_bf16(x32, lib=rnd)
    assert np.array_equal(got, ref), "bf16 rounding"


MIXER_PINS = [pin_conv_torch, pin_conv_delta_taps, pin_mixer_torch, pin_round_bf16_matches_torch]


# ------------------------------------------------------------------------------------------
# P-10 (continuation): initial states drawn from a pool by index, and the conv input window
# carried from one call to the next (a prefix hands its conv window and recurrent state to each
# candidate).  Each takes ``api`` with the callables fwd, fwd_idx, conv_cont, mixer_cont
# (signatures of oracle.gdn_fwd, gdn_fwd_indexed, conv_silu_cont, mixer_fwd_cont).
# ------------------------------------------------------------------------------------------
def pin_fanout_brute(api, d=3, seed=41):
    """Exact rational brute force per sequence with S_0 = pool[index] (zero when out of range)."""
    from oracle import brute
    rng = np.random.default_rng(seed)
    R = lambda: Fraction(int(rng.integers(-8, 9)), 8)
    lengths = [3, 2, 0, 4, 2]
    index = [1, 1, 0, -1, 5]  # repeated, an empty sequence, negative and past-the-end indices
    pool = [[[R() for _ in range(d)] for _ in range(d)] for _ in range(2)]  # value-major S_0
    T = sum(lengths)
    alpha = [Fraction(int(rng.integers(1, 9)), 8) for _ in range(T)]
    beta = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    q = [[R() for _ in range(d)] for _ in range(T)]
    k = [[R() for _ in range(d)] for _ in range(T)]
    v = [[R() for _ in range(d)] for _ in range(T)]
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    h0 = np.stack([f(S).T for S in pool])[:, None]  # [2, 1, d, d] key-major
    o, hT = api.fwd_idx(f(q)[:, None], f(k)[:, None], f(v)[:, None],
                        np.log(np.array([float(a) for a in alpha]))[:, None],
                        np.array([float(b) for b in beta])[:, None], cu, h0, index)
    zero = [[Fraction(0)] * d for _ in range(d)]
    for n, L in enumerate(lengths):
        S0 = pool[index[n]] if 0 <= index[n] < 2 else zero
        sl = slice(cu[n], cu[n + 1])
        if L == 0:  # an empty sequence hands its initial state through
            assert np.array_equal(hT[n, 0], f(S0).T), "fan-out hT (empty sequence)"
            continue
        outs, ST = brute.run(alpha[sl], beta[sl], q[sl], k[sl], v[sl], S0)
        assert np.allclose(o[sl, 0], f(outs), rtol=1e-12, atol=1e-13), "fan-out o"
        assert np.allclose(hT[n, 0], f(ST).T, rtol=1e-12, atol=1e-13), "fan-out hT"


def pin_fanout_equals_gathered(api):
    """Indexing the pool equals handing each sequence an explicit copy (bitwise)."""
    rng = np.random.default_rng(42)
    q, k, v, g, beta, cu, _ = _rand_case(rng, 0, 2, 4, 8, lengths=[9, 70, 0, 5, 33], h0=False)
    pool = rng.standard_normal((3, 4, 8, 8)) * 0.3
    index = np.array([2, 0, 2, 3, 2])  # index 3 is outside the pool: zero state
    o, hT = api.fwd_idx(q, k, v, g, beta, cu, pool, index)
    gathered = np.stack([pool[i] if 0 <= i < 3 else np.zeros((4, 8, 8)) for i in index])
    o2, h2 = api.fwd(q, k, v, g, beta, cu, gathered)
    assert np.array_equal(o, o2) and np.array_equal(hT, h2), "fan-out vs copies"


def pin_conv_window_numpy(api):
    """Conv over (window ++ tokens) against numpy's correlate; the window out is the stream's last
    taps-1 entries -- for sequences shorter than the window too."""
    rng = np.random.default_rng(43)
    C, taps = 6, 4
    lengths = [0, 1, 2, 3, 9]
    index = np.array([2, 0, -1, 0, 7])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    x = rng.standard_normal((cu[-1], C))
    w = 0.5 * rng.standard_normal((C, taps))
    pool = rng.standard_normal((3, taps - 1, C))
    out, wout = api.conv_cont(x, w, cu, pool, index)
    for n in range(len(lengths)):
        win = pool[index[n]] if 0 <= index[n] < 3 else np.zeros((taps - 1, C))
        stream = np.concatenate([win, x[cu[n]:cu[n + 1]]])
        for ch in range(C if lengths[n] else 0):
            c = np.correlate(stream[:, ch], w[ch], mode="valid")
            assert np.allclose(out[cu[n]:cu[n + 1], ch], c / (1 + np.exp(-c)), rtol=1e-12, atol=1e-13), "conv window"
        assert np.array_equal(wout[n], stream[-(taps - 1):]), "window out"


def _mixer_case(rng, lengths, Hk=2, Hv=4, d=8):
    T = sum(lengths)
    C = 2 * Hk * d + Hv * d
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(qkv=rng.standard_normal((T, C)), conv_w=0.5 * rng.standard_normal((C, 4)),
                g=-np.log1p(np.exp(-(3 + rng.standard_normal((T, Hv))))),
                beta=1 / (1 + np.exp(-rng.standard_normal((T, Hv)))), z=rng.standard_normal((T, Hv, d)),
                norm_w=1 + 0.1 * rng.standard_normal(d), cu=cu, Hk=Hk, Hv=Hv, d=d)


def _mix(api, m, sl_tok, cu, h0, conv_in, index, points):
    return api.mixer_cont(m["qkv"][sl_tok], m["conv_w"], m["g"][sl_tok], m["beta"][sl_tok], m["z"][sl_tok],
                          m["norm_w"], cu, h0, conv_in, index, Hk=m["Hk"], Hv=m["Hv"], dk=m["d"], dv=m["d"],
                          bf16_points=points)


def pin_mixer_split_continuation(api):
    """Two sequences, each cut at s: running the tails from the heads' states and windows equals
    one run of the whole sequences (bitwise, with and without the bf16 points)."""
    rng = np.random.default_rng(44)
    m = _mixer_case(rng, [13, 21])
    L = [13, 21]
    h0 = 0.1 * rng.standard_normal((2, m["Hv"], m["d"], m["d"]))
    for points in (False, True):
        y, hT, wout = _mix(api, m, slice(None), m["cu"], h0, None, None, points)
        for s in (1, 2, 7):
            head = np.concatenate([np.arange(s), 13 + np.arange(s)])
            tail = np.concatenate([np.arange(s, 13), 13 + np.arange(s, 21)])
            ya, ha, wa = _mix(api, m, head, [0, s, 2 * s], h0, None, None, points)
            yb, hb, wb = _mix(api, m, tail, [0, 13 - s, 34 - 2 * s], ha, wa, None, points)
            yy = np.zeros_like(y)
            yy[head], yy[tail] = ya, yb
            assert np.array_equal(yy, y), f"mixer continuation y (split {s})"
            assert np.array_equal(hb, hT) and np.array_equal(wb, wout), f"mixer continuation state (split {s})"


def pin_mixer_fanout(api):
    """Indexed pools of states and windows equal explicitly gathered copies (bitwise)."""
    rng = np.random.default_rng(45)
    m = _mixer_case(rng, [5, 0, 17, 2])
    C = m["qkv"].shape[1]
    h0 = 0.1 * rng.standard_normal((2, m["Hv"], m["d"], m["d"]))
    win = rng.standard_normal((2, 3, C))
    index = np.array([1, 1, -1, 0])
    y, hT, wout = _mix(api, m, slice(None), m["cu"], h0, win, index, True)
    gh = np.stack([h0[i] if 0 <= i < 2 else np.zeros_like(h0[0]) for i in index])
    gw = np.stack([win[i] if 0 <= i < 2 else np.zeros_like(win[0]) for i in index])
    y2, h2, w2 = _mix(api, m, slice(None), m["cu"], gh, gw, None, True)
    assert np.array_equal(y, y2) and np.array_equal(hT, h2) and np.array_equal(wout, w2), "mixer fan-out"


CONT_PINS = [pin_fanout_brute, pin_fanout_equals_gathered, pin_conv_window_numpy, pin_mixer_split_continuation,
             pin_mixer_fanout]


# ------------------------------------------------------------------------------------------
# Gate parameters: g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b) per token and v-head.
# Each takes ``gates`` (signature of oracle.gates).
# ------------------------------------------------------------------------------------------
def pin_gates_closed_forms(gates):
    # a + dt_bias = 0: softplus(0) = ln 2, so g = -exp(A_log) ln 2; b = 0: beta = 1/2 exactly
    A_log = np.array([0.0, np.log(2.0), -1.5, 2.0])
    dt = np.array([0.25, -3.0, 1.0, 0.0])
    g, beta = gates(np.tile(-dt, (3, 1)), np.zeros((3, 4)), A_log, dt)
    assert np.allclose(g, -np.exp(A_log) * np.log(2.0), rtol=1e-15, atol=0), "g at softplus(0)"
    assert np.array_equal(beta, np.full((3, 4), 0.5)), "beta at b = 0"
    # with A_log = dt_bias = 0: softplus(x) - softplus(-x) = x and sigmoid(x) + sigmoid(-x) = 1
    x = np.random.default_rng(61).standard_normal((5, 4)) * 4.0
    z4 = np.zeros(4)
    gp, bp = gates(x, x, z4, z4)
    gm, bm = gates(-x, -x, z4, z4)
    assert np.allclose(gm - gp, x, rtol=0, atol=1e-13), "softplus(x) - softplus(-x) = x"
    assert np.allclose(bp + bm, 1.0, rtol=0, atol=1e-15), "sigmoid(x) + sigmoid(-x) = 1"
    assert np.all(gp < 0) and np.all((bp > 0) & (bp < 1)), "g < 0 < beta < 1"


def pin_gates_library(gates):
    # against numpy's logaddexp (softplus) and scipy's expit (sigmoid), with |x| up to 60
    from scipy.special import expit
    rng = np.random.default_rng(62)
    T, Hv = 40, 6
    a = rng.standard_normal((T, Hv)) * 3.0
    b = rng.standard_normal((T, Hv)) * 3.0
    a[0], b[0] = 60.0, -60.0
    a[1], b[1] = -60.0, 60.0
    A_log = rng.uniform(-1.0, 2.8, Hv)
    dt = np.log(np.expm1(rng.uniform(1e-3, 0.1, Hv)))
    g, beta = gates(a, b, A_log, dt)
    assert np.allclose(g, -np.exp(A_log) * np.logaddexp(0.0, a + dt), rtol=1e-14, atol=1e-300), "g vs logaddexp"
    assert np.allclose(beta, expit(b), rtol=1e-14, atol=1e-300), "beta vs expit"


GATE_PINS = [pin_gates_closed_forms, pin_gates_library]
