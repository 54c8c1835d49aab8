"""fp64 CPU oracle for the chunked Gated DeltaNet path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.

* :func:`gdn_fwd` -- the gated delta rule token by token in fp64 (plain C +
  OpenMP over (sequence, v-head) pairs, ``gdn_oracle.c``); :func:`gdn_fwd_indexed`
  draws each sequence's initial state from a pool by index (one prefix state handed
  to several candidates, "open-jev-fast" README, "Phase 2" item 2).  The recurrence is
  the Gated DeltaNet rule that the "open-jev-fast" README ("Phase 3", item 1,
  reference [5]) implements in chunked form:
  ``S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T``,
  ``o_t = S_t q_t``, over packed variable-length sequences each with its own
  optional initial state (System1-Omni PR #186, "Purpose and summary").
* :func:`mixer_fwd` -- conv + SiLU, q/k L2 norm, the rule, SiLU(z)-gated RMSNorm
  ("open-jev-fast" README, "Phase 2", item 1); :func:`mixer_fwd_cont` also carries
  the conv input window in and out beside the recurrent state, so that a call
  continues where another stopped.
* :func:`gates` -- the gate parameters g and beta from the layer's projections (the last
  input-prep step the "open-jev-fast" README, "Phase 2" item 1, names; the pages give no
  formula, so it follows the Mamba2-style gating of the Gated DeltaNet paper that README cites).
* :mod:`oracle.brute` -- exact rational arithmetic for tiny cases.

State layout: ``h0``/``hT`` are key-major ``[N, Hv, dk, dv]`` (``H = S^T``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain IEEE fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open an oracle shared library built from ``gdn_oracle.c`` (or a test's mutant of it)."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_gdn_fwd.argtypes = [i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, i32]
    lib.oracle_gdn_fwd.restype = ctypes.c_int
    lib.oracle_gdn_fwd_indexed.argtypes = [i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, i32, P,
                                           P, P, i32]
    lib.oracle_gdn_fwd_indexed.restype = ctypes.c_int
    lib.oracle_conv_silu.argtypes = [i64, i32, i32, i32, P, P, P, P, i32]
    lib.oracle_conv_silu.restype = ctypes.c_int
    lib.oracle_conv_silu_cont.argtypes = [i64, i32, i32, i32, P, P, P, P, i32, P, P, P, i32]
    lib.oracle_conv_silu_cont.restype = ctypes.c_int
    lib.oracle_mixer_fwd.argtypes = [i64, i32, i32, i32, i32, i32, i32, f64, f64, i32,
                                     P, P, P, P, P, P, P, P, P, P, i32]
    lib.oracle_mixer_fwd_cont.argtypes = [i64, i32, i32, i32, i32, i32, i32, f64, f64, i32,
                                          P, P, P, P, P, P, P, P, P, i32, P, P, P, P, i32]
    lib.oracle_mixer_fwd_cont.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [f64]
    lib.oracle_round_bf16.restype = f64
    lib.oracle_round_bf16_array.argtypes = [P, P, i64]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_mixer_fwd.restype = ctypes.c_int
    lib.oracle_gates.argtypes = [i64, i32, P, P, P, P, P, P]
    lib.oracle_gates.restype = None
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = load_library(_LIB)
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cu(cu, T):
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing, start at 0 and end at T")
    return cu


def gdn_fwd(q, k, v, g, beta, cu_seqlens, h0=None, threads: int = 0, want_state: bool = True, lib=None):
    """Token-by-token gated delta rule in fp64.

    q, k: [T, Hk, dk]; v: [T, Hv, dv]; g, beta: [T, Hv]; cu_seqlens: [N+1];
    h0: [N, Hv, dk, dv] or None.  Returns (o [T, Hv, dv], hT [N, Hv, dk, dv]).
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, Hv) or beta.shape != (T, Hv):
        raise ValueError("shape mismatch")
    if h0 is not None:
        h0 = _f64(h0)
        if h0.shape != (N, Hv, dk, dv):
            raise ValueError("h0 shape")
    o = np.zeros((T, Hv, dv))
    hT = np.zeros((N, Hv, dk, dv)) if want_state else None
    rc = (lib or _load()).oracle_gdn_fwd(T, N, Hk, Hv, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(cu), _ptr(h0), _ptr(o), _ptr(hT), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdn_fwd failed ({rc})")
    return o, hT


def conv_silu(x, w, cu_seqlens, threads: int = 0, lib=None):
    """Causal depthwise conv (taps = w.shape[1]) + SiLU, per sequence. x: [T, C]; w: [C, taps]."""
    x, w = _f64(x), _f64(w)
    T, C = x.shape
    cu = _cu(cu_seqlens, T)
    out = np.zeros((T, C))
    rc = (lib or _load()).oracle_conv_silu(T, cu.size - 1, C, w.shape[1], _ptr(x), _ptr(w), _ptr(cu), _ptr(out),
                                  int(threads))
    if rc != 0:
        raise RuntimeError("oracle_conv_silu failed")
    return out


def _index(idx, N):
    if idx is None:
        return None
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64))
    if idx.shape != (N,):
        raise ValueError("index shape")
    return idx


def gdn_fwd_indexed(q, k, v, g, beta, cu_seqlens, h0, h0_index, threads: int = 0, want_state: bool = True,
                    lib=None):
    """The rule with sequence n starting from ``h0[h0_index[n]]`` (a zero state when the index is
    outside ``[0, len(h0))``).  h0: [num_h0, Hv, dk, dv]; h0_index: [N] integers."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    h0 = _f64(h0)
    if h0.ndim != 4 or h0.shape[1:] != (Hv, dk, dv) or h0.shape[0] < 1:
        raise ValueError("h0 shape")
    idx = _index(h0_index, N)
    o = np.zeros((T, Hv, dv))
    hT = np.zeros((N, Hv, dk, dv)) if want_state else None
    rc = (lib or _load()).oracle_gdn_fwd_indexed(T, N, Hk, Hv, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                                 _ptr(beta), _ptr(cu), _ptr(h0), h0.shape[0], _ptr(idx),
                                                 _ptr(o), _ptr(hT), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdn_fwd_indexed failed ({rc})")
    return o, hT


def conv_silu_cont(x, w, cu_seqlens, win_in=None, state_index=None, threads: int = 0, lib=None):
    """Conv + SiLU continuing from carried input windows.  win_in: [num_states, taps-1, C] or None
    (zeros); state_index: [N] or None (window n).  Returns (out [T, C], win_out [N, taps-1, C])."""
    x, w = _f64(x), _f64(w)
    T, C = x.shape
    taps = w.shape[1]
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    idx = _index(state_index, N)
    ns = N
    if win_in is not None:
        win_in = _f64(win_in)
        if win_in.ndim != 3 or win_in.shape[1:] != (taps - 1, C):
            raise ValueError("window shape")
        ns = win_in.shape[0]
    out = np.zeros((T, C))
    win_out = np.zeros((N, taps - 1, C))
    rc = (lib or _load()).oracle_conv_silu_cont(T, N, C, taps, _ptr(x), _ptr(w), _ptr(cu), _ptr(win_in), ns,
                                                _ptr(idx), _ptr(out), _ptr(win_out), int(threads))
    if rc != 0:
        raise RuntimeError("oracle_conv_silu_cont failed")
    return out, win_out


def round_bf16(x, lib=None):
    """Round fp64 values to bf16 (8 significant bits, ties to even), elementwise."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(a)
    (lib or _load()).oracle_round_bf16_array(_ptr(a), _ptr(out), a.size)
    return out


def gates(a, b, A_log, dt_bias, lib=None):
    """Gate parameters in fp64: g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b), per token
    and v-head.  a, b: [T, Hv]; A_log, dt_bias: [Hv].  Returns (g, beta), each [T, Hv]."""
    a, b, A_log, dt_bias = (_f64(x) for x in (a, b, A_log, dt_bias))
    if a.ndim != 2 or b.shape != a.shape or A_log.shape != (a.shape[1],) or dt_bias.shape != A_log.shape:
        raise ValueError("gate shapes")
    g = np.empty_like(a)
    beta = np.empty_like(a)
    (lib or _load()).oracle_gates(a.shape[0], a.shape[1], _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(g),
                                  _ptr(beta))
    return g, beta


def mixer_fwd(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0=None, Hk=16, Hv=32, dk=128, dv=128,
              eps_l2=1e-6, eps_norm=1e-6, bf16_points: bool = True, threads: int = 0, lib=None):
    """Full GDN mixer in fp64. Returns (y [T, Hv, dv], hT [N, Hv, dk, dv]).

    bf16_points: round the prepped q, k, v and the rule's output o to bf16 where the bf16 model
    does ("open-jev-fast" README, "Phase 2" item 1); all other arithmetic is fp64."""
    qkv, conv_w, g, beta, z, norm_w = (_f64(x) for x in (qkv, conv_w, g, beta, z, norm_w))
    T = qkv.shape[0]
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    if qkv.shape[1] != 2 * Hk * dk + Hv * dv or conv_w.shape[0] != qkv.shape[1]:
        raise ValueError("channel mismatch")
    if h0 is not None:
        h0 = _f64(h0)
    y = np.zeros((T, Hv, dv))
    hT = np.zeros((N, Hv, dk, dv))
    rc = (lib or _load()).oracle_mixer_fwd(T, N, Hk, Hv, dk, dv, conv_w.shape[1], float(eps_l2), float(eps_norm),
                                  int(bool(bf16_points)), _ptr(qkv), _ptr(conv_w), _ptr(g), _ptr(beta), _ptr(z), _ptr(norm_w),
                                  _ptr(cu), _ptr(h0), _ptr(y), _ptr(hT), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_mixer_fwd failed ({rc})")
    return y, hT


def mixer_fwd_cont(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0=None, conv_in=None, state_index=None,
                   Hk=16, Hv=32, dk=128, dv=128, eps_l2=1e-6, eps_norm=1e-6, bf16_points: bool = True,
                   threads: int = 0, lib=None):
    """The mixer continuing from carried states: sequence n starts from recurrent state and conv
    window ``state_index[n]`` of the pools h0 [S, Hv, dk, dv] and conv_in [S, taps-1, C] (zeros for
    an index outside [0, S), or for a pool that is None; None index means state n).
    Returns (y [T, Hv, dv], hT [N, Hv, dk, dv], conv_out [N, taps-1, C])."""
    qkv, conv_w, g, beta, z, norm_w = (_f64(x) for x in (qkv, conv_w, g, beta, z, norm_w))
    T, C = qkv.shape
    taps = conv_w.shape[1]
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    if C != 2 * Hk * dk + Hv * dv or conv_w.shape[0] != C:
        raise ValueError("channel mismatch")
    idx = _index(state_index, N)
    sizes = set()
    if h0 is not None:
        h0 = _f64(h0)
        sizes.add(h0.shape[0])
    if conv_in is not None:
        conv_in = _f64(conv_in)
        if conv_in.shape[1:] != (taps - 1, C):
            raise ValueError("window shape")
        sizes.add(conv_in.shape[0])
    if len(sizes) > 1:
        raise ValueError("h0 and conv_in pools differ in size")
    ns = sizes.pop() if sizes else N
    y = np.zeros((T, Hv, dv))
    hT = np.zeros((N, Hv, dk, dv))
    conv_out = np.zeros((N, taps - 1, C))
    rc = (lib or _load()).oracle_mixer_fwd_cont(T, N, Hk, Hv, dk, dv, taps, float(eps_l2), float(eps_norm),
                                                int(bool(bf16_points)), _ptr(qkv), _ptr(conv_w), _ptr(g),
                                                _ptr(beta), _ptr(z), _ptr(norm_w), _ptr(cu), _ptr(h0),
                                                _ptr(conv_in), ns, _ptr(idx), _ptr(y), _ptr(hT),
                                                _ptr(conv_out), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_mixer_fwd_cont failed ({rc})")
    return y, hT, conv_out
