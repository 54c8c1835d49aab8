"""The C ABI on the host, without a GPU: the library loads, exports every symbol include/gdn.h
declares, and rejects every invalid argument with its status code before anything is enqueued.
No call here reaches a kernel launch (all arguments are invalid by construction)."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_deltanet_chunked_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"GDN_EXPORT\s+[\w\s\*]+?\b(gdn_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_symbols() == sorted(gdn.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [s for s in declared_symbols() if s not in exported]
    assert not missing, f"not exported: {missing}"
    # nothing else with C linkage leaks out under the gdn_ prefix
    extra = sorted(s for s in exported if s.startswith("gdn_") and s not in declared_symbols())
    assert not extra, f"undeclared exports: {extra}"


def test_abi_version_and_status_strings():
    assert gdn.gdn_abi_version() == 1
    m = re.search(r"#define GDN_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == gdn.gdn_abi_version()
    names = ["GDN_OK", "GDN_ERR_NULL", "GDN_ERR_SHAPE", "GDN_ERR_UNSUPPORTED", "GDN_ERR_ALIGN",
             "GDN_ERR_WORKSPACE", "GDN_ERR_ALIAS", "GDN_ERR_HIP", "GDN_ERR_SCRATCH_LIMIT"]
    for code, name in enumerate(names):
        assert gdn.gdn_status_string(code).startswith(name)
    assert "unknown" in gdn.gdn_status_string(99)
    assert gdn.gdn_last_hip_error() == 0


def test_workspace_size():
    # slots = T // 64 + N; per slot: Hv records of 18944 B (256-aligned); a single sequence of at
    # least 32 chunks with at most 8 v-heads adds three buffers of 32 fp32 128 x 128 states (the
    # time split)
    def expect(T, N, Hk, Hv):
        r = lambda x: (x + 255) // 256 * 256
        s = T // 64 + N
        split = 3 * 32 * 128 * 128 * 4 if (N == 1 and Hv <= 8 and T > 31 * 64) else 0
        return r(s * Hv * 18944) + split
    for args in [(16384, 1, 16, 32), (677, 7, 16, 32), (0, 1, 4, 4), (1, 3, 1, 2), (16384, 1, 2, 4),
                 (1984, 1, 1, 8), (1985, 1, 1, 8), (1985, 1, 1, 16), (1985, 2, 1, 8)]:
        assert gdn.gdn_chunk_fwd_workspace_size(*args) == expect(*args), args
    assert gdn.gdn_chunk_fwd_workspace_size(10, 1, 3, 4) == 0     # Hv % Hk != 0
    assert gdn.gdn_chunk_fwd_workspace_size(10, 0, 1, 1) == 0     # N < 1
    assert gdn.gdn_chunk_fwd_workspace_size(-1, 1, 1, 1) == 0     # T < 0
    d = gdn.ChunkDesc(10, 1, 1, 1, 64, 128, None, 0)
    assert gdn.lib().gdn_chunk_fwd_workspace_size(ctypes.byref(d)) == 0   # dk != 128
    mix = gdn.gdn_mixer_fwd_workspace_size(936, 1, 16, 32)
    assert mix > gdn.gdn_chunk_fwd_workspace_size(936, 1, 16, 32)
    assert gdn.gdn_mixer_fwd_workspace_size(936, 1, 16, 32, conv_taps=3) == 0


# ---------------------------------------------------------------------------------------------
# Validation: fake, well-separated device addresses; every call must fail before any launch.
# ---------------------------------------------------------------------------------------------
T, N, HK, HV = 100, 1, 2, 4
GB = 1 << 30


def _addrs():
    # distinct 1 GiB-spaced, 256-aligned fake addresses (never dereferenced)
    base = 0x7F0000000000
    names = ["q", "k", "v", "g", "beta", "cu", "h0", "o", "hT", "ws"]
    return {n: base + i * GB for i, n in enumerate(names)}


def _call(desc=None, **over):
    a = _addrs()
    a.update(over)
    ws_bytes = gdn.gdn_chunk_fwd_workspace_size(T, N, HK, HV)
    d = desc if desc is not None else gdn.ChunkDesc(T, N, HK, HV, 128, 128, a["ws"], ws_bytes)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return gdn.lib().gdn_chunk_fwd(ctypes.byref(d) if d is not False else None, P(a["q"]), P(a["k"]), P(a["v"]),
                                   P(a["g"]), P(a["beta"]), P(a["cu"]), P(a["h0"]), P(a["o"]), P(a["hT"]), None)


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "beta", "cu", "o"])
def test_null_pointers(field):
    assert _call(**{field: None}) == gdn.GDN_ERR_NULL


def test_null_descriptor():
    assert _call(desc=False) == gdn.GDN_ERR_NULL


def test_bad_shapes():
    a = _addrs()
    ws = gdn.gdn_chunk_fwd_workspace_size(T, N, HK, HV)
    for bad in [gdn.ChunkDesc(T, 0, HK, HV, 128, 128, a["ws"], ws), gdn.ChunkDesc(-5, N, HK, HV, 128, 128, a["ws"], ws),
                gdn.ChunkDesc(T, N, 3, HV, 128, 128, a["ws"], ws), gdn.ChunkDesc(T, N, 0, HV, 128, 128, a["ws"], ws)]:
        assert _call(desc=bad) == gdn.GDN_ERR_SHAPE
    for bad in [gdn.ChunkDesc(T, N, HK, HV, 64, 128, a["ws"], ws), gdn.ChunkDesc(T, N, HK, HV, 128, 256, a["ws"], ws)]:
        assert _call(desc=bad) == gdn.GDN_ERR_UNSUPPORTED


def test_workspace_checks():
    a = _addrs()
    ws = gdn.gdn_chunk_fwd_workspace_size(T, N, HK, HV)
    assert _call(desc=gdn.ChunkDesc(T, N, HK, HV, 128, 128, a["ws"], ws - 1)) == gdn.GDN_ERR_WORKSPACE
    assert _call(desc=gdn.ChunkDesc(T, N, HK, HV, 128, 128, None, ws)) == gdn.GDN_ERR_WORKSPACE


@pytest.mark.parametrize("field,off", [("q", 8), ("k", 2), ("v", 4), ("o", 8), ("h0", 4), ("hT", 12),
                                       ("g", 2), ("beta", 1), ("cu", 2)])
def test_alignment(field, off):
    a = _addrs()
    assert _call(**{field: a[field] + off}) == gdn.GDN_ERR_ALIGN


def test_alignment_of_workspace():
    a = _addrs()
    ws = gdn.gdn_chunk_fwd_workspace_size(T, N, HK, HV)
    assert _call(desc=gdn.ChunkDesc(T, N, HK, HV, 128, 128, a["ws"] + 8, ws)) == gdn.GDN_ERR_ALIGN


def test_aliasing():
    a = _addrs()
    assert _call(o=a["q"]) == gdn.GDN_ERR_ALIAS                 # output over an input
    assert _call(o=a["v"] + 1024) == gdn.GDN_ERR_ALIAS          # partial overlap
    assert _call(hT=a["o"]) == gdn.GDN_ERR_ALIAS                # two outputs overlap
    assert _call(hT=a["h0"] + 256) == gdn.GDN_ERR_ALIAS         # partial overlap with h0
    assert _call(ws=a["k"]) == gdn.GDN_ERR_ALIAS                # workspace over an input


def test_workspace_alias_with_input():
    a = _addrs()
    ws = gdn.gdn_chunk_fwd_workspace_size(T, N, HK, HV)
    assert _call(desc=gdn.ChunkDesc(T, N, HK, HV, 128, 128, a["k"], ws)) == gdn.GDN_ERR_ALIAS


@pytest.mark.parametrize("entry", ["gdn_mixer_fwd", "gdn_mixer_fwd_fused_norm"])
def test_mixer_validation(entry):
    # the fused-norm entry point checks its arguments exactly as gdn_mixer_fwd does, before it looks
    # at the device (whether the work fits in one round) or launches anything
    a = _addrs()
    ws = gdn.gdn_mixer_fwd_workspace_size(T, N, HK, HV)
    P = ctypes.c_void_p
    fn = getattr(gdn.lib(), entry)

    def call(m, **over):
        b = {"qkv": a["q"], "cw": a["k"], "g": a["g"], "beta": a["beta"], "z": a["v"], "nw": a["h0"] + GB // 2,
             "cu": a["cu"], "h0": a["h0"], "y": a["o"], "hT": a["hT"]}
        b.update(over)
        pp = lambda x: None if x is None else P(x)
        return fn(ctypes.byref(m) if m is not None else None, pp(b["qkv"]), pp(b["cw"]), pp(b["g"]), pp(b["beta"]),
                  pp(b["z"]), pp(b["nw"]), pp(b["cu"]), pp(b["h0"]), pp(b["y"]), pp(b["hT"]), None)

    assert call(None) == gdn.GDN_ERR_NULL

    good = lambda taps=4, eps=1e-6, wsb=ws: gdn.MixerDesc(gdn.ChunkDesc(T, N, HK, HV, 128, 128, a["ws"], wsb), taps, eps)
    assert call(good(taps=3)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(good(eps=0.0)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(good(wsb=ws - 1)) == gdn.GDN_ERR_WORKSPACE
    assert call(good(), z=None) == gdn.GDN_ERR_NULL
    assert call(good(), cw=a["k"] + 4) == gdn.GDN_ERR_ALIGN
    assert call(good(), nw=a["h0"] + GB // 2 + 4) == gdn.GDN_ERR_ALIGN
    assert call(good(), y=a["v"]) == gdn.GDN_ERR_ALIAS          # y over z
    # T * Hv rows of the gated RMSNorm beyond one grid of 16-row blocks
    big = gdn.MixerDesc(gdn.ChunkDesc(2 ** 31 - 256, 1, 1, 32, 128, 128, a["ws"], ws), 4, 1e-6)
    assert gdn.gdn_mixer_fwd_workspace_size(2 ** 31 - 256, 1, 1, 32) == 0
    assert call(big) == gdn.GDN_ERR_SHAPE


def test_mixer_gates_validation():
    # the gates entry point: gdn_mixer_fwd's checks, with a, b (bf16 [T, Hv]) and A_log, dt_bias
    # (fp32 [Hv]) in place of g and beta; every check runs before anything is launched
    a = _addrs()
    ws = gdn.gdn_mixer_fwd_workspace_size(T, N, HK, HV)
    P = ctypes.c_void_p
    fn = gdn.lib().gdn_mixer_fwd_gates

    def call(m, **over):
        b = {"qkv": a["q"], "cw": a["k"], "ga": a["g"], "gb": a["beta"], "A_log": a["cu"] + GB // 2,
             "dt": a["cu"] + GB // 2 + 256, "z": a["v"], "nw": a["h0"] + GB // 2, "cu": a["cu"], "h0": a["h0"],
             "y": a["o"], "hT": a["hT"]}
        b.update(over)
        pp = lambda x: None if x is None else P(x)
        return fn(ctypes.byref(m) if m is not None else None, pp(b["qkv"]), pp(b["cw"]), pp(b["ga"]), pp(b["gb"]),
                  pp(b["A_log"]), pp(b["dt"]), pp(b["z"]), pp(b["nw"]), pp(b["cu"]), pp(b["h0"]), pp(b["y"]),
                  pp(b["hT"]), None)

    good = lambda wsb=ws: gdn.MixerDesc(gdn.ChunkDesc(T, N, HK, HV, 128, 128, a["ws"], wsb), 4, 1e-6)
    assert call(None) == gdn.GDN_ERR_NULL
    for field in ("ga", "gb", "A_log", "dt"):
        assert call(good(), **{field: None}) == gdn.GDN_ERR_NULL, field
    assert call(good(wsb=ws - 1)) == gdn.GDN_ERR_WORKSPACE
    assert call(good(), ga=a["g"] + 1) == gdn.GDN_ERR_ALIGN
    assert call(good(), gb=a["beta"] + 1) == gdn.GDN_ERR_ALIGN
    assert call(good(), A_log=a["cu"] + GB // 2 + 2) == gdn.GDN_ERR_ALIGN
    assert call(good(), dt=a["cu"] + GB // 2 + 258) == gdn.GDN_ERR_ALIGN
    assert call(good(), y=a["g"]) == gdn.GDN_ERR_ALIAS          # y over a
    assert call(good(), hT=a["cu"] + GB // 2) == gdn.GDN_ERR_ALIAS  # hT over A_log


def _call_indexed(num_h0=3, idx=None, **over):
    a = _addrs()
    a["idx"] = a["cu"] + GB // 2
    a.update(over)
    if idx is not None:
        a["idx"] = idx
    ws_bytes = gdn.gdn_chunk_fwd_workspace_size(T, N, HK, HV)
    d = gdn.ChunkDesc(T, N, HK, HV, 128, 128, a["ws"], ws_bytes)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return gdn.lib().gdn_chunk_fwd_indexed(ctypes.byref(d), P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]),
                                           P(a["beta"]), P(a["cu"]), P(a["h0"]), num_h0, P(a["idx"]), P(a["o"]),
                                           P(a["hT"]), None)


def test_indexed_validation():
    a = _addrs()
    row = HV * 128 * 128 * 4
    idx = a["cu"] + GB // 2
    assert _call_indexed(h0=None) == gdn.GDN_ERR_NULL           # a pool is required
    assert _call_indexed(idx=0) == gdn.GDN_ERR_NULL             # NULL index
    assert _call_indexed(num_h0=0) == gdn.GDN_ERR_SHAPE
    assert _call_indexed(num_h0=-2) == gdn.GDN_ERR_SHAPE
    assert _call_indexed(idx=idx + 2) == gdn.GDN_ERR_ALIGN
    assert _call_indexed(h0=a["h0"] + 4) == gdn.GDN_ERR_ALIGN
    assert _call_indexed(hT=a["h0"]) == gdn.GDN_ERR_ALIAS       # no in-place with an index
    assert _call_indexed(hT=a["h0"] + 2 * row) == gdn.GDN_ERR_ALIAS   # row 2 of a 3-row pool
    assert _call_indexed(o=idx - 256) == gdn.GDN_ERR_ALIAS      # o over the index
    assert _call_indexed(q=None) == gdn.GDN_ERR_NULL


def test_mixer_cont_validation():
    a = _addrs()
    ws = gdn.gdn_mixer_fwd_workspace_size(T, N, HK, HV)
    C = (2 * HK + HV) * 128
    P = ctypes.c_void_p
    extra = a["cu"] + GB // 2  # room for the index and the windows, each under 1 MiB

    def call(S=N, **over):
        b = {"qkv": a["q"], "cw": a["k"], "g": a["g"], "beta": a["beta"], "z": a["v"], "nw": a["h0"] + GB // 2,
             "cu": a["cu"], "h0": a["h0"], "cin": extra, "idx": None, "y": a["o"], "hT": a["hT"],
             "cout": extra + (1 << 20)}
        b.update(over)
        pp = lambda x: None if x is None else P(x)
        m = gdn.MixerDesc(gdn.ChunkDesc(T, N, HK, HV, 128, 128, a["ws"], ws), 4, 1e-6)
        return gdn.lib().gdn_mixer_fwd_cont(ctypes.byref(m), pp(b["qkv"]), pp(b["cw"]), pp(b["g"]), pp(b["beta"]),
                                            pp(b["z"]), pp(b["nw"]), pp(b["cu"]), pp(b["h0"]), pp(b["cin"]), S,
                                            pp(b["idx"]), pp(b["y"]), pp(b["hT"]), pp(b["cout"]), None)

    idx = extra + (2 << 20)
    assert call(S=2) == gdn.GDN_ERR_SHAPE                        # pool size must be N without an index
    assert call(S=0, idx=idx) == gdn.GDN_ERR_SHAPE
    assert call(cin=extra + 8) == gdn.GDN_ERR_ALIGN
    assert call(cout=extra + (1 << 20) + 4) == gdn.GDN_ERR_ALIGN
    assert call(S=2, idx=idx + 1) == gdn.GDN_ERR_ALIGN
    assert call(S=2, idx=idx, cout=extra) == gdn.GDN_ERR_ALIAS  # in-place window with an index
    assert call(S=2, idx=idx, hT=a["h0"]) == gdn.GDN_ERR_ALIAS  # in-place state with an index
    assert call(cout=extra + 3 * C) == gdn.GDN_ERR_ALIAS         # partial overlap with conv_in
    assert call(cout=a["o"]) == gdn.GDN_ERR_ALIAS                # two outputs overlap
    assert call(y=idx, S=2, idx=idx) == gdn.GDN_ERR_ALIAS        # y over the index
    assert call(z=None) == gdn.GDN_ERR_NULL


def test_mixer_gates_cont_validation():
    # the continued mixer with its gates made in the first kernel: gdn_mixer_fwd_cont's checks with
    # gdn_mixer_fwd_gates's in place of those of g and beta; every check runs before any launch
    a = _addrs()
    ws = gdn.gdn_mixer_fwd_workspace_size(T, N, HK, HV)
    P = ctypes.c_void_p
    extra = a["cu"] + GB // 2  # windows, index and the per-head gate parameters, each under 1 MiB

    def call(S=N, **over):
        b = {"qkv": a["q"], "cw": a["k"], "ga": a["g"], "gb": a["beta"], "A_log": extra + (3 << 20),
             "dt": extra + (3 << 20) + 256, "z": a["v"], "nw": a["h0"] + GB // 2, "cu": a["cu"], "h0": a["h0"],
             "cin": extra, "idx": None, "y": a["o"], "hT": a["hT"], "cout": extra + (1 << 20)}
        b.update(over)
        pp = lambda x: None if x is None else P(x)
        m = gdn.MixerDesc(gdn.ChunkDesc(T, N, HK, HV, 128, 128, a["ws"], ws), 4, 1e-6)
        return gdn.lib().gdn_mixer_fwd_gates_cont(
            ctypes.byref(m), pp(b["qkv"]), pp(b["cw"]), pp(b["ga"]), pp(b["gb"]), pp(b["A_log"]), pp(b["dt"]),
            pp(b["z"]), pp(b["nw"]), pp(b["cu"]), pp(b["h0"]), pp(b["cin"]), S, pp(b["idx"]), pp(b["y"]),
            pp(b["hT"]), pp(b["cout"]), None)

    idx = extra + (2 << 20)
    assert call(S=2) == gdn.GDN_ERR_SHAPE                        # pool size must be N without an index
    for field in ("ga", "gb", "A_log", "dt"):
        assert call(**{field: None}) == gdn.GDN_ERR_NULL, field
    assert call(ga=a["g"] + 1) == gdn.GDN_ERR_ALIGN
    assert call(dt=extra + (3 << 20) + 258) == gdn.GDN_ERR_ALIGN
    assert call(cin=extra + 8) == gdn.GDN_ERR_ALIGN
    assert call(S=2, idx=idx, cout=extra) == gdn.GDN_ERR_ALIAS  # in-place window with an index
    assert call(cout=a["g"]) == gdn.GDN_ERR_ALIAS                # window out over a
    assert call(hT=extra + (3 << 20)) == gdn.GDN_ERR_ALIAS       # hT over A_log
    assert call(z=None) == gdn.GDN_ERR_NULL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gdn, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(gdn, "_lib_handle", None)
    with pytest.raises(RuntimeError, match="missing"):
        gdn.gdn_abi_version()


def test_noalloc_scratch_limit():
    # The scratch limit is checked on the host before the static scratch is looked up or anything
    # is launched: a shape whose workspace exceeds it is rejected, an invalid shape keeps its own
    # status, and the limit in the header matches the binding's.
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == gdn.NOALLOC_SCRATCH_BYTES
    L = gdn.lib()
    a = _addrs()
    args = [ctypes.c_void_p(a[n]) for n in ("q", "k", "v", "g", "beta", "cu", "h0", "o", "hT")] + [None]
    for (T_, N_, Hk_, Hv_) in [(7040, 1, 16, 32), (16384, 1, 16, 32), (64 * 1000, 1, 1, 4)]:
        assert gdn.gdn_chunk_fwd_workspace_size(T_, N_, Hk_, Hv_) > gdn.NOALLOC_SCRATCH_BYTES
        d = gdn.ChunkDesc(T_, N_, Hk_, Hv_, 128, 128, None, 0)
        rc = L.gdn_chunk_fwd_noalloc(ctypes.byref(d), *args)
        assert rc == gdn.GDN_ERR_SCRATCH_LIMIT, (T_, rc)
    assert gdn.gdn_chunk_fwd_workspace_size(7039, 1, 16, 32) <= gdn.NOALLOC_SCRATCH_BYTES
    d = gdn.ChunkDesc(10, 1, 3, 4, 128, 128, None, 0)  # Hv % Hk != 0
    assert L.gdn_chunk_fwd_noalloc(ctypes.byref(d), *args) == gdn.GDN_ERR_SHAPE
    assert L.gdn_chunk_fwd_noalloc(None, *args) == gdn.GDN_ERR_NULL


def test_binding_cu_seqlens_host_check():
    # The binding checks a host copy of cu_seqlens before any call (the library cannot read it
    # without a sync): short ones as a Python list, long ones with numpy; every input form.
    import numpy as np
    import torch

    T = 936
    ok = [[0, T], (0, 0, T), torch.tensor([0, T], dtype=torch.int64), torch.tensor([0, 100, T], dtype=torch.int32),
          np.array([0, 5, 5, T]), torch.arange(0, T + 1, dtype=torch.int64), np.arange(0, T + 1)]
    for host in ok:
        assert gdn._check_cu(None, T, host) == len(host) - 1
    long_bad = torch.arange(0, T + 1, dtype=torch.int64)
    long_bad[500] = 3  # not monotone, past the short-list path
    bad = [[0, 5, 3, T], [1, T], [0, T - 1], [0], [], [[0, T]], torch.tensor([[0, T]]), torch.tensor([0, 7, 2, T]),
           long_bad, long_bad.numpy()]
    for host in bad:
        with pytest.raises(ValueError):
            gdn._check_cu(None, T, host)


def test_plan_argument_checks():
    # ChunkPlan and MixerPlan check every argument on the host when they are made; nothing is
    # launched here (forward() is never called).  Valid arguments give outputs of the right shapes;
    # each kind of mistake raises.  The tensors are CPU tensors: the checks only ask that all of a
    # call's tensors share one device.
    import torch

    T, Hk, Hv, D = 100, 2, 4, 128
    bf, f32 = torch.bfloat16, torch.float32
    cu_h = [0, 40, T]
    c = dict(q=torch.zeros((T, Hk, D), dtype=bf), k=torch.zeros((T, Hk, D), dtype=bf),
             v=torch.zeros((T, Hv, D), dtype=bf), g=torch.zeros((T, Hv), dtype=f32),
             beta=torch.zeros((T, Hv), dtype=f32), cu_seqlens=torch.tensor(cu_h, dtype=torch.int32))

    def chunk(**kw):
        a = dict(c, **kw)
        host = a.pop("cu_seqlens_host", cu_h)
        return gdn.ChunkPlan(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"], a.get("h0"),
                             workspace=a.get("workspace"), cu_seqlens_host=host)

    p = chunk()
    assert p.o.shape == (T, Hv, D) and p.o.dtype == bf and p.hT.shape == (2, Hv, D, D)
    assert p.workspace.numel() == gdn.gdn_chunk_fwd_workspace_size(T, 2, Hk, Hv)
    bad = [(TypeError, dict(g=c["g"].double())),
           (ValueError, dict(beta=c["beta"][:-1])),
           (ValueError, dict(v=torch.zeros((T, Hv, 2 * D), dtype=bf)[..., :D])),  # not contiguous
           (ValueError, dict(h0=torch.zeros((1, Hv, D, D), dtype=f32))),  # one state for two sequences
           (TypeError, dict(cu_seqlens=c["cu_seqlens"].long())),
           (ValueError, dict(cu_seqlens_host=[0, 60, 40, T])),
           (ValueError, dict(workspace=torch.zeros(16, dtype=torch.uint8))),
           (gdn.GdnError, dict(v=torch.zeros((T, 3, D), dtype=bf), g=torch.zeros((T, 3), dtype=f32),
                               beta=torch.zeros((T, 3), dtype=f32)))]  # Hv not a multiple of Hk
    for exc, kw in bad:
        with pytest.raises(exc):
            chunk(**kw)

    C = (2 * Hk + Hv) * D
    m = dict(qkv=torch.zeros((T, C), dtype=bf), conv_w=torch.zeros((C, 4), dtype=bf), g=c["g"], beta=c["beta"],
             z=torch.zeros((T, Hv, D), dtype=bf), norm_w=torch.ones(D, dtype=bf), cu_seqlens=c["cu_seqlens"])

    def mixer(gates=None, want_state=True, **kw):
        a = dict(m, **kw)
        return gdn.MixerPlan(a["qkv"], a["conv_w"], a["g"], a["beta"], a["z"], a["norm_w"], a["cu_seqlens"],
                             a.get("h0"), Hk=a.get("Hk", Hk), Hv=Hv, want_state=want_state, cu_seqlens_host=cu_h,
                             gates=gates)

    p = mixer()
    assert p.y.shape == (T, Hv, D) and p.hT.shape == (2, Hv, D, D)
    assert mixer(want_state=False).hT is None
    gates = (torch.zeros((T, Hv), dtype=bf), torch.zeros((T, Hv), dtype=bf), torch.zeros(Hv, dtype=f32),
             torch.zeros(Hv, dtype=f32))
    assert mixer(gates=gates, g=None, beta=None).y.shape == (T, Hv, D)
    bad = [(ValueError, dict(qkv=torch.zeros((T, C - D), dtype=bf))),
           (TypeError, dict(z=torch.zeros((T, Hv, D), dtype=f32))),
           (ValueError, dict(conv_w=torch.zeros((C, 3), dtype=bf))),
           (ValueError, dict(h0=torch.zeros((2, Hv, D, 64), dtype=f32))),
           (TypeError, dict(gates=(gates[0].float(),) + gates[1:], g=None, beta=None)),
           (ValueError, dict(gates=gates[:2] + (torch.zeros(Hv + 1, dtype=f32), gates[3]), g=None, beta=None)),
           (ValueError, dict(Hk=3))]  # qkv's width no longer matches (2 Hk + Hv) 128
    for exc, kw in bad:
        with pytest.raises(exc):
            mixer(**kw)
