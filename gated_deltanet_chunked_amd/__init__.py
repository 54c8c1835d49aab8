"""Python binding of libgdn -- chunked Gated DeltaNet prefill forward on AMD MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels behind the C ABI
declared in ``include/gdn.h``.  PyTorch supplies device memory and the stream; there is no CPU or
PyTorch fallback.  If ``libgdn.so`` has not been built, every entry point raises.

Entry points (same names as the C ABI):
    gdn_abi_version(), gdn_status_string(code), gdn_last_hip_error()
    gdn_chunk_fwd_workspace_size(T, N, Hk, Hv)
    gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens, h0=None, ...) -> (o, hT)
    gdn_chunk_fwd_indexed(q, k, v, g, beta, cu_seqlens, h0, h0_index, ...) -> (o, hT)
    gdn_chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens, h0, o=..., hT=...): gdn_chunk_fwd on the
        library's static scratch, for callers that cannot allocate (outputs passed in)
    gdn_chunk_prep / gdn_state_pass: the two stages of gdn_chunk_fwd (see ChunkPlan)
    gdn_mixer_fwd_workspace_size(T, N, Hk, Hv)
    gdn_mixer_fwd(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0=None, ...) -> (y, hT)
    gdn_mixer_fwd_cont(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0, conv_in, state_index, ...)
        -> (y, hT, conv_out)
    gdn_mixer_fwd_gates / gdn_mixer_fwd_gates_cont: the same with g and beta made from the
        projections a, b and the per-head A_log, dt_bias
    gdn_mixer_fwd_fused_norm: gdn_mixer_fwd with the gated RMSNorm inside the state pass
ChunkPlan and MixerPlan check one call's arguments once, for repeated calls on fixed buffers
(forward() then costs only the C call and its launches).

Layouts (row-major, contiguous): q, k bf16 [T, Hk, 128]; v bf16 [T, Hv, 128]; g, beta fp32
[T, Hv]; cu_seqlens int32 [N+1]; h0, hT fp32 [N, Hv, 128, 128] key-major (H = S^T); o bf16
[T, Hv, 128].  See ``include/gdn.h`` for the full contract.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
D = 128

GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED = 0, 1, 2, 3
GDN_ERR_ALIGN, GDN_ERR_WORKSPACE, GDN_ERR_ALIAS, GDN_ERR_HIP = 4, 5, 6, 7
GDN_ERR_SCRATCH_LIMIT = 8
NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES

EXPORTED_SYMBOLS = ("gdn_abi_version", "gdn_status_string", "gdn_last_hip_error",
                    "gdn_chunk_fwd_workspace_size", "gdn_chunk_fwd", "gdn_chunk_fwd_indexed",
                    "gdn_chunk_fwd_noalloc", "gdn_chunk_prep",
                    "gdn_state_pass", "gdn_mixer_fwd_workspace_size", "gdn_mixer_fwd", "gdn_mixer_fwd_cont",
                    "gdn_mixer_fwd_fused_norm", "gdn_mixer_fwd_gates", "gdn_mixer_fwd_gates_cont")


class ChunkDesc(ctypes.Structure):
    _fields_ = [("total_tokens", ctypes.c_int64), ("num_seqs", ctypes.c_int32),
                ("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class MixerDesc(ctypes.Structure):
    _fields_ = [("chunk", ChunkDesc), ("conv_taps", ctypes.c_int32), ("norm_eps", ctypes.c_float)]


class GdnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = f"{where}: {gdn_status_string(code)}"
        if code == GDN_ERR_HIP:
            msg += f" (hipError {gdn_last_hip_error()})"
        super().__init__(msg)


_lib_handle = None


def lib():
    """The loaded libgdn.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gated_deltanet_chunked_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        L.gdn_abi_version.restype = ctypes.c_int
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_last_hip_error.restype = ctypes.c_int
        L.gdn_chunk_fwd_workspace_size.restype = S
        L.gdn_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(ChunkDesc)]
        L.gdn_chunk_fwd.restype = ctypes.c_int
        L.gdn_chunk_fwd.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 10
        L.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
        L.gdn_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 10
        L.gdn_chunk_fwd_indexed.restype = ctypes.c_int
        L.gdn_chunk_fwd_indexed.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 7 + [ctypes.c_int32] + [P] * 4
        L.gdn_chunk_prep.restype = ctypes.c_int
        L.gdn_chunk_prep.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 6
        L.gdn_state_pass.restype = ctypes.c_int
        L.gdn_state_pass.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 8
        L.gdn_mixer_fwd_workspace_size.restype = S
        L.gdn_mixer_fwd_workspace_size.argtypes = [ctypes.POINTER(MixerDesc)]
        L.gdn_mixer_fwd.restype = ctypes.c_int
        L.gdn_mixer_fwd.argtypes = [ctypes.POINTER(MixerDesc)] + [P] * 11
        L.gdn_mixer_fwd_fused_norm.restype = ctypes.c_int
        L.gdn_mixer_fwd_fused_norm.argtypes = [ctypes.POINTER(MixerDesc)] + [P] * 11
        L.gdn_mixer_fwd_gates.restype = ctypes.c_int
        L.gdn_mixer_fwd_gates.argtypes = [ctypes.POINTER(MixerDesc)] + [P] * 13
        L.gdn_mixer_fwd_cont.restype = ctypes.c_int
        L.gdn_mixer_fwd_cont.argtypes = [ctypes.POINTER(MixerDesc)] + [P] * 9 + [ctypes.c_int32] + [P] * 5
        L.gdn_mixer_fwd_gates_cont.restype = ctypes.c_int
        L.gdn_mixer_fwd_gates_cont.argtypes = [ctypes.POINTER(MixerDesc)] + [P] * 11 + [ctypes.c_int32] + [P] * 5
        _lib_handle = L
    return _lib_handle


def gdn_abi_version() -> int:
    return int(lib().gdn_abi_version())


def gdn_status_string(code: int) -> str:
    return lib().gdn_status_string(int(code)).decode()


def gdn_last_hip_error() -> int:
    return int(lib().gdn_last_hip_error())


def _desc(T, N, Hk, Hv, ws=None, ws_bytes=0, dk=D, dv=D) -> ChunkDesc:
    return ChunkDesc(int(T), int(N), int(Hk), int(Hv), int(dk), int(dv), ws, int(ws_bytes))


def gdn_chunk_fwd_workspace_size(T: int, N: int, Hk: int, Hv: int) -> int:
    return _chunk_ws_size(int(T), int(N), int(Hk), int(Hv))


def gdn_mixer_fwd_workspace_size(T: int, N: int, Hk: int, Hv: int, conv_taps: int = 4,
                                 norm_eps: float = 1e-6) -> int:
    return _mixer_ws_size(int(T), int(N), int(Hk), int(Hv), int(conv_taps), float(norm_eps))


# The sizes depend on the shape alone; the calls ask for them every time, so they are kept.
@functools.lru_cache(maxsize=256)
def _chunk_ws_size(T, N, Hk, Hv):
    return int(lib().gdn_chunk_fwd_workspace_size(ctypes.byref(_desc(T, N, Hk, Hv))))


@functools.lru_cache(maxsize=256)
def _mixer_ws_size(T, N, Hk, Hv, conv_taps, norm_eps):
    m = MixerDesc(_desc(T, N, Hk, Hv), conv_taps, norm_eps)
    return int(lib().gdn_mixer_fwd_workspace_size(ctypes.byref(m)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape, device):
    if t.dtype is dtype and t.shape == shape and t.is_contiguous() and t.device == device:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _check_cu(cu_seqlens, T, cu_host):
    # Plain Python or numpy on the host copy: small torch operations here cost ~16 us a call, as
    # much as the rest of a mixer call's host work.
    host = cu_host if cu_host is not None else cu_seqlens.detach().cpu()
    if isinstance(host, torch.Tensor):
        host = host.detach().cpu()
        a = host.tolist() if host.dim() == 1 and host.numel() <= 64 else host.numpy()
    else:
        a = np.asarray(host)
    if isinstance(a, list):
        ok = len(a) >= 2 and a[0] == 0 and a[-1] == T and all(x <= y for x, y in zip(a, a[1:]))
    else:
        ok = a.ndim == 1 and a.size >= 2 and int(a[0]) == 0 and int(a[-1]) == T and not bool(np.any(a[1:] < a[:-1]))
    if not ok:
        raise ValueError("cu_seqlens must be non-decreasing, start at 0 and end at T")
    return len(a) - 1


def _torch_stream(stream, device):
    """The stream to enqueue on as a torch stream: the given one (a torch stream or a raw
    hipStream_t handle), else the current stream of the tensors' device."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _stream(stream, device):
    return ctypes.c_void_p(_torch_stream(stream, device).cuda_stream)


def _keep_for(stream, device, tensors):
    """Tensors this binding allocated for a call that runs on a stream other than the current
    one: tell the caching allocator they are in use on that stream, so that once the caller drops
    them their memory is not handed to a new allocation on the current stream while the call's
    kernels may still be reading or writing it."""
    if stream is None or not any(t is not None for t in tensors):
        return  # on the current stream itself, or nothing allocated here
    ts = _torch_stream(stream, device)
    if ts != torch.cuda.current_stream(device):
        for t in tensors:
            if t is not None:
                t.record_stream(ts)


def _workspace(workspace, need, device, fresh):
    """A caller's workspace (uint8, contiguous, on the device, at least `need` bytes), or a new one
    (appended to `fresh`, the tensors allocated for this call)."""
    if workspace is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        fresh.append(ws)
        return ws
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != device:
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    return workspace


def _chunk_io(q, k, v, g, beta, cu_seqlens, o, hT, want_state, workspace, cu_seqlens_host):
    dev = q.device
    T, Hk = int(q.shape[0]), int(q.shape[1])
    Hv = int(v.shape[1])
    _check(q, "q", torch.bfloat16, (T, Hk, D), dev)
    _check(k, "k", torch.bfloat16, (T, Hk, D), dev)
    _check(v, "v", torch.bfloat16, (T, Hv, D), dev)
    _check(g, "g", torch.float32, (T, Hv), dev)
    _check(beta, "beta", torch.float32, (T, Hv), dev)
    N = _check_cu(cu_seqlens, T, cu_seqlens_host)
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    fresh = []
    if o is None:
        o = torch.empty((T, Hv, D), dtype=torch.bfloat16, device=dev)
        fresh.append(o)
    _check(o, "o", torch.bfloat16, (T, Hv, D), dev)
    if hT is None and want_state:
        hT = torch.empty((N, Hv, D, D), dtype=torch.float32, device=dev)
        fresh.append(hT)
    if hT is not None:
        _check(hT, "hT", torch.float32, (N, Hv, D, D), dev)
    need = gdn_chunk_fwd_workspace_size(T, N, Hk, Hv)
    if need == 0:
        raise GdnError(GDN_ERR_SHAPE, "gdn_chunk_fwd_workspace_size")
    workspace = _workspace(workspace, need, dev, fresh)
    return T, N, Hk, Hv, o, hT, _desc(T, N, Hk, Hv, workspace.data_ptr(), workspace.numel()), fresh


def gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens, h0=None, *, o=None, hT=None, want_state=True,
                  workspace=None, stream=None, cu_seqlens_host=None):
    """Chunked gated-delta-rule forward.  Returns (o, hT) (hT is None if not wanted).

    ``cu_seqlens_host`` (a CPU copy) avoids the device sync of checking ``cu_seqlens``.
    ``workspace`` (uint8 CUDA tensor) may be passed to avoid an allocation per call.
    """
    T, N, Hk, Hv, o, hT, d, fresh = _chunk_io(q, k, v, g, beta, cu_seqlens, o, hT, want_state, workspace,
                                              cu_seqlens_host)
    if h0 is not None:
        _check(h0, "h0", torch.float32, (N, Hv, D, D), q.device)
    rc = lib().gdn_chunk_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                             _ptr(h0), _ptr(o), _ptr(hT), _stream(stream, q.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd")
    _keep_for(stream, q.device, fresh)
    return o, hT


def gdn_chunk_fwd_indexed(q, k, v, g, beta, cu_seqlens, h0, h0_index, *, o=None, hT=None, want_state=True,
                          workspace=None, stream=None, cu_seqlens_host=None):
    """gdn_chunk_fwd with sequence n starting from ``h0[h0_index[n]]`` of a pool of initial states
    (h0: fp32 [num_h0, Hv, 128, 128]; h0_index: int32 [N] on the device; an index outside
    [0, num_h0) means a zero state).  One prefix state fans out to many candidates without copies.
    hT may not overlap h0.  Returns (o, hT)."""
    T, N, Hk, Hv, o, hT, d, fresh = _chunk_io(q, k, v, g, beta, cu_seqlens, o, hT, want_state, workspace,
                                              cu_seqlens_host)
    if h0.dim() != 4 or h0.shape[0] < 1:
        raise ValueError("h0 must be [num_h0, Hv, 128, 128] with num_h0 >= 1")
    _check(h0, "h0", torch.float32, (int(h0.shape[0]), Hv, D, D), q.device)
    _check(h0_index, "h0_index", torch.int32, (N,), q.device)
    rc = lib().gdn_chunk_fwd_indexed(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(cu_seqlens), _ptr(h0), int(h0.shape[0]), _ptr(h0_index), _ptr(o),
                                     _ptr(hT), _stream(stream, q.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd_indexed")
    _keep_for(stream, q.device, fresh)
    return o, hT


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens, h0=None, *, o, hT=None, stream=None,
                          cu_seqlens_host=None):
    """gdn_chunk_fwd on the library's static device scratch instead of a workspace, for callers
    that cannot allocate: the outputs o (bf16 [T, Hv, 128]) and, if wanted, hT (fp32
    [N, Hv, 128, 128]) are passed in, and nothing is allocated here or in the library.  Shapes
    whose workspace would exceed NOALLOC_SCRATCH_BYTES raise GdnError(GDN_ERR_SCRATCH_LIMIT).
    Calls that overlap in time on one GPU share the scratch and race; order them on one stream.
    Returns (o, hT)."""
    dev = q.device
    T, Hk, Hv = int(q.shape[0]), int(q.shape[1]), int(v.shape[1])
    _check(q, "q", torch.bfloat16, (T, Hk, D), dev)
    _check(k, "k", torch.bfloat16, (T, Hk, D), dev)
    _check(v, "v", torch.bfloat16, (T, Hv, D), dev)
    _check(g, "g", torch.float32, (T, Hv), dev)
    _check(beta, "beta", torch.float32, (T, Hv), dev)
    N = _check_cu(cu_seqlens, T, cu_seqlens_host)
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    _check(o, "o", torch.bfloat16, (T, Hv, D), dev)
    if hT is not None:
        _check(hT, "hT", torch.float32, (N, Hv, D, D), dev)
    if h0 is not None:
        _check(h0, "h0", torch.float32, (N, Hv, D, D), dev)
    d = _desc(T, N, Hk, Hv)
    rc = lib().gdn_chunk_fwd_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(cu_seqlens), _ptr(h0), _ptr(o), _ptr(hT), _stream(stream, dev))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd_noalloc")
    return o, hT


class ChunkPlan:
    """Checked arguments of one gdn_chunk_fwd call on fixed buffers: forward() runs the whole call,
    prep() and state_pass() its two stages (e.g. to time each kernel on its own).  The tensors are
    bound when the plan is made (their pointers are kept); write new data into them between calls
    rather than replacing them."""

    def __init__(self, q, k, v, g, beta, cu_seqlens, h0=None, *, o=None, hT=None, workspace=None,
                 cu_seqlens_host=None):
        dev = q.device
        T, Hk, Hv = int(q.shape[0]), int(q.shape[1]), int(v.shape[1])
        _check(q, "q", torch.bfloat16, (T, Hk, D), dev)
        _check(k, "k", torch.bfloat16, (T, Hk, D), dev)
        _check(v, "v", torch.bfloat16, (T, Hv, D), dev)
        _check(g, "g", torch.float32, (T, Hv), dev)
        _check(beta, "beta", torch.float32, (T, Hv), dev)
        N = _check_cu(cu_seqlens, T, cu_seqlens_host)
        _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
        if h0 is not None:
            _check(h0, "h0", torch.float32, (N, Hv, D, D), dev)
        self._fresh = []
        self.o = o
        if o is None:
            self.o = torch.empty((T, Hv, D), dtype=torch.bfloat16, device=dev)
            self._fresh.append(self.o)
        self.hT = hT
        if hT is None:
            self.hT = torch.empty((N, Hv, D, D), dtype=torch.float32, device=dev)
            self._fresh.append(self.hT)
        _check(self.o, "o", torch.bfloat16, (T, Hv, D), dev)
        _check(self.hT, "hT", torch.float32, (N, Hv, D, D), dev)
        need = gdn_chunk_fwd_workspace_size(T, N, Hk, Hv)
        if need == 0:
            raise GdnError(GDN_ERR_SHAPE, "gdn_chunk_fwd_workspace_size")
        self.workspace = _workspace(workspace, need, dev, self._fresh)
        self.device = dev
        self.desc = _desc(T, N, Hk, Hv, self.workspace.data_ptr(), self.workspace.numel())
        self.args = (q, k, v, g, beta, cu_seqlens, h0)
        # the plan's tensors keep their addresses: their pointer arguments are made once
        self._desc_ref = ctypes.byref(self.desc)
        pq, pk, pv, pg, pb, pcu, ph0 = (_ptr(t) for t in self.args)
        self._prep_args = (pq, pk, pg, pb, pcu)
        self._pass_args = (pq, pk, pv, pcu, ph0, _ptr(self.o), _ptr(self.hT))
        self._fwd_args = (pq, pk, pv, pg, pb, pcu, ph0, _ptr(self.o), _ptr(self.hT))

    def prep(self, stream=None):
        rc = lib().gdn_chunk_prep(self._desc_ref, *self._prep_args, _stream(stream, self.device))
        if rc != GDN_OK:
            raise GdnError(rc, "gdn_chunk_prep")
        _keep_for(stream, self.device, self._fresh)

    def state_pass(self, stream=None):
        rc = lib().gdn_state_pass(self._desc_ref, *self._pass_args, _stream(stream, self.device))
        if rc != GDN_OK:
            raise GdnError(rc, "gdn_state_pass")
        _keep_for(stream, self.device, self._fresh)

    def forward(self, stream=None):
        rc = lib().gdn_chunk_fwd(self._desc_ref, *self._fwd_args, _stream(stream, self.device))
        if rc != GDN_OK:
            raise GdnError(rc, "gdn_chunk_fwd")
        _keep_for(stream, self.device, self._fresh)


def gdn_mixer_fwd(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0=None, *, Hk=16, Hv=32, y=None, hT=None,
                  want_state=True, norm_eps=1e-6, workspace=None, stream=None, cu_seqlens_host=None,
                  fused_norm=False):
    """GDN mixer forward (conv + SiLU + L2 norm, the chunked rule, gated RMSNorm).  Returns (y, hT).
    fused_norm=True calls gdn_mixer_fwd_fused_norm (the norm inside the state pass; slower on
    MI355X, and GdnError(GDN_ERR_UNSUPPORTED) where the work items do not fit in one round)."""
    y, hT, _ = _mixer(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0, None, None, False, Hk, Hv, y, hT, None,
                      want_state, False, norm_eps, workspace, stream, cu_seqlens_host, fused_norm)
    return y, hT


def gdn_mixer_fwd_gates(qkv, conv_w, a, b, A_log, dt_bias, z, norm_w, cu_seqlens, h0=None, *, Hk=16, Hv=32,
                        y=None, hT=None, want_state=True, norm_eps=1e-6, workspace=None, stream=None,
                        cu_seqlens_host=None):
    """gdn_mixer_fwd with the gate parameters made in the mixer's first kernel from the projections:
    g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b) per token and v-head.  a, b: bf16
    [T, Hv]; A_log, dt_bias: fp32 [Hv].  Returns (y, hT)."""
    y, hT, _ = _mixer(qkv, conv_w, None, None, z, norm_w, cu_seqlens, h0, None, None, False, Hk, Hv, y, hT, None,
                      want_state, False, norm_eps, workspace, stream, cu_seqlens_host, False,
                      gates=(a, b, A_log, dt_bias))
    return y, hT


def gdn_mixer_fwd_gates_cont(qkv, conv_w, a, b, A_log, dt_bias, z, norm_w, cu_seqlens, h0=None, conv_in=None,
                             state_index=None, *, Hk=16, Hv=32, y=None, hT=None, conv_out=None, want_state=True,
                             want_window=True, norm_eps=1e-6, workspace=None, stream=None, cu_seqlens_host=None):
    """gdn_mixer_fwd_cont with the gate parameters made in the mixer's first kernel, as in
    gdn_mixer_fwd_gates.  Returns (y, hT, conv_out)."""
    return _mixer(qkv, conv_w, None, None, z, norm_w, cu_seqlens, h0, conv_in, state_index, True, Hk, Hv, y, hT,
                  conv_out, want_state, want_window, norm_eps, workspace, stream, cu_seqlens_host, False,
                  gates=(a, b, A_log, dt_bias))


def gdn_mixer_fwd_cont(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0=None, conv_in=None, state_index=None, *,
                       Hk=16, Hv=32, y=None, hT=None, conv_out=None, want_state=True, want_window=True,
                       norm_eps=1e-6, workspace=None, stream=None, cu_seqlens_host=None):
    """The mixer continuing from carried states: sequence n starts from recurrent state and conv
    window ``state_index[n]`` (int32 [N] on the device; None = state n) of the pools h0 (fp32
    [S, Hv, 128, 128]) and conv_in (bf16 [S, 3, C], the last 3 qkv rows before the sequence,
    oldest first); either pool may be None (zeros).  Returns (y, hT, conv_out) with conv_out bf16
    [N, 3, C], the window the next call continues from."""
    return _mixer(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0, conv_in, state_index, True, Hk, Hv, y, hT,
                  conv_out, want_state, want_window, norm_eps, workspace, stream, cu_seqlens_host)


def _mixer_call(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0, conv_in, state_index, cont, Hk, Hv, y, hT,
                conv_out, want_state, want_window, norm_eps, workspace, cu_seqlens_host, fused_norm=False, gates=None):
    """Checks a mixer call's arguments and allocates the outputs and workspace not given.  Returns
    (C function, its name, its arguments but the stream, (y, hT, conv_out), tensors allocated)."""
    dev = qkv.device
    T = int(qkv.shape[0])
    C = (2 * Hk + Hv) * D
    _check(qkv, "qkv", torch.bfloat16, (T, C), dev)
    _check(conv_w, "conv_w", torch.bfloat16, (C, 4), dev)
    if gates is None:
        _check(g, "g", torch.float32, (T, Hv), dev)
        _check(beta, "beta", torch.float32, (T, Hv), dev)
    else:
        ga, gb, A_log, dt_bias = gates
        _check(ga, "a", torch.bfloat16, (T, Hv), dev)
        _check(gb, "b", torch.bfloat16, (T, Hv), dev)
        _check(A_log, "A_log", torch.float32, (Hv,), dev)
        _check(dt_bias, "dt_bias", torch.float32, (Hv,), dev)
    _check(z, "z", torch.bfloat16, (T, Hv, D), dev)
    _check(norm_w, "norm_w", torch.bfloat16, (D,), dev)
    N = _check_cu(cu_seqlens, T, cu_seqlens_host)
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    S = N
    if state_index is not None:
        _check(state_index, "state_index", torch.int32, (N,), dev)
        pools = [int(t.shape[0]) for t in (h0, conv_in) if t is not None]
        if len(set(pools)) > 1:
            raise ValueError("h0 and conv_in pools must have the same number of states")
        S = pools[0] if pools else 1
    if h0 is not None:
        _check(h0, "h0", torch.float32, (S, Hv, D, D), dev)
    if conv_in is not None:
        _check(conv_in, "conv_in", torch.bfloat16, (S, 3, C), dev)
    fresh = []
    if y is None:
        y = torch.empty((T, Hv, D), dtype=torch.bfloat16, device=dev)
        fresh.append(y)
    _check(y, "y", torch.bfloat16, (T, Hv, D), dev)
    if hT is None and want_state:
        hT = torch.empty((N, Hv, D, D), dtype=torch.float32, device=dev)
        fresh.append(hT)
    if hT is not None:
        _check(hT, "hT", torch.float32, (N, Hv, D, D), dev)
    if conv_out is None and cont and want_window:
        conv_out = torch.empty((N, 3, C), dtype=torch.bfloat16, device=dev)
        fresh.append(conv_out)
    if conv_out is not None:
        _check(conv_out, "conv_out", torch.bfloat16, (N, 3, C), dev)
    need = gdn_mixer_fwd_workspace_size(T, N, Hk, Hv, 4, norm_eps)
    if need == 0:
        raise GdnError(GDN_ERR_SHAPE, "gdn_mixer_fwd_workspace_size")
    workspace = _workspace(workspace, need, dev, fresh)
    m = MixerDesc(_desc(T, N, Hk, Hv, workspace.data_ptr(), workspace.numel()), 4, float(norm_eps))
    ref = ctypes.byref(m)
    if cont and gates is not None:
        fn, where = lib().gdn_mixer_fwd_gates_cont, "gdn_mixer_fwd_gates_cont"
        args = (ref, _ptr(qkv), _ptr(conv_w), _ptr(ga), _ptr(gb), _ptr(A_log), _ptr(dt_bias), _ptr(z), _ptr(norm_w),
                _ptr(cu_seqlens), _ptr(h0), _ptr(conv_in), S, _ptr(state_index), _ptr(y), _ptr(hT), _ptr(conv_out))
    elif cont:
        fn, where = lib().gdn_mixer_fwd_cont, "gdn_mixer_fwd_cont"
        args = (ref, _ptr(qkv), _ptr(conv_w), _ptr(g), _ptr(beta), _ptr(z), _ptr(norm_w), _ptr(cu_seqlens), _ptr(h0),
                _ptr(conv_in), S, _ptr(state_index), _ptr(y), _ptr(hT), _ptr(conv_out))
    elif gates is not None:
        fn, where = lib().gdn_mixer_fwd_gates, "gdn_mixer_fwd_gates"
        args = (ref, _ptr(qkv), _ptr(conv_w), _ptr(ga), _ptr(gb), _ptr(A_log), _ptr(dt_bias), _ptr(z), _ptr(norm_w),
                _ptr(cu_seqlens), _ptr(h0), _ptr(y), _ptr(hT))
    else:
        fn, where = ((lib().gdn_mixer_fwd_fused_norm, "gdn_mixer_fwd_fused_norm") if fused_norm
                     else (lib().gdn_mixer_fwd, "gdn_mixer_fwd"))
        args = (ref, _ptr(qkv), _ptr(conv_w), _ptr(g), _ptr(beta), _ptr(z), _ptr(norm_w), _ptr(cu_seqlens), _ptr(h0),
                _ptr(y), _ptr(hT))
    return fn, where, args, (y, hT, conv_out), fresh


def _mixer(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0, conv_in, state_index, cont, Hk, Hv, y, hT, conv_out,
           want_state, want_window, norm_eps, workspace, stream, cu_seqlens_host, fused_norm=False, gates=None):
    fn, where, args, outs, fresh = _mixer_call(qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0, conv_in, state_index,
                                               cont, Hk, Hv, y, hT, conv_out, want_state, want_window, norm_eps,
                                               workspace, cu_seqlens_host, fused_norm, gates)
    dev = qkv.device
    rc = fn(*args, _stream(stream, dev))
    if rc != GDN_OK:
        raise GdnError(rc, where)
    _keep_for(stream, dev, fresh)
    return outs


class MixerPlan:
    """Checked arguments of one gdn_mixer_fwd call on fixed buffers (gdn_mixer_fwd_gates with
    gates=(a, b, A_log, dt_bias), g and beta then None); forward() runs it and returns (y, hT).
    The tensors are bound when the plan is made (their pointers are kept); write new data into
    them between calls rather than replacing them."""

    def __init__(self, qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0=None, *, Hk=16, Hv=32, y=None, hT=None,
                 want_state=True, norm_eps=1e-6, workspace=None, cu_seqlens_host=None, gates=None):
        self.device = qkv.device
        self._fn, self._where, self._args, outs, self._fresh = _mixer_call(
            qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0, None, None, False, Hk, Hv, y, hT, None, want_state,
            False, norm_eps, workspace, cu_seqlens_host, False, gates)
        self.y, self.hT, _ = outs
        self._keep = (qkv, conv_w, g, beta, z, norm_w, cu_seqlens, h0, gates, workspace)

    def forward(self, stream=None):
        rc = self._fn(*self._args, _stream(stream, self.device))
        if rc != GDN_OK:
            raise GdnError(rc, self._where)
        _keep_for(stream, self.device, self._fresh)
        return self.y, self.hT
