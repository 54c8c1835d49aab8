"""Seeded synthetic inputs for the chunked Gated DeltaNet path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no part of the method's arithmetic: it only draws random numbers with
numpy's PCG64 and rounds them to the storage types (bf16 round-to-nearest-even
as raw uint16 bits, fp32, int32).  Both the HIP path and the fp64 oracle get
exactly the stored values.

Workload shapes and distributions (the pages' workloads, stood in for by
synthetic data; the pages' own benchmark requests are not used):
  * lengths 256, 539, 936, 3,399, 16,384 tokens, a 7-sequence packed batch
    (the "open-jev-fast" README: 539-token example with 7 candidates and a
    16,384 max length; the H200 blog, "Gated DeltaNet preparation -- PR #68":
    GDN calls at 936 and 3,399 tokens);
  * Hk = 16 q/k heads, Hv = 32 v heads, d = 128 ("open-jev-fast" README,
    "Phase 3" item 3, q/k at 16 heads);
  * q, k ~ N(0,1) L2-normalised per (token, head); v ~ N(0,1);
    beta = sigmoid(N(0,1)); g = log(sigmoid(N(3,1))) = -log1p(exp(-x));
    initial states ~ 0.05 N(0,1) (second parameter read as a std-dev).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

D = 128


def bf16_bits(x) -> np.ndarray:
    """Round to bf16 (round-to-nearest-even via fp32) and return the uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(f)
    out = r.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def bits_to_f64(bits) -> np.ndarray:
    return bits_to_f32(bits).astype(np.float64)


@dataclass
class GdnCase:
    name: str
    Hk: int
    Hv: int
    lengths: List[int]
    seed: int
    with_h0: bool = False
    h0_std: float = 0.05
    g_mean: float = 3.0

    @property
    def T(self) -> int:
        return int(sum(self.lengths))

    @property
    def N(self) -> int:
        return len(self.lengths)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)


# The five workloads of the measurement plan (sizes named by what they are).
CASES = {
    "t256_h4": GdnCase("t256_h4", 4, 4, [256], seed=1),
    "t539_h16x32": GdnCase("t539_h16x32", 16, 32, [539], seed=2),
    "varlen7_t677_h0": GdnCase("varlen7_t677_h0", 16, 32, [61, 73, 88, 95, 104, 117, 139], seed=3,
                               with_h0=True),
    # the mixer layer's shape (T = 936) with the distributions of the rule's own inputs above
    "t936_h16x32": GdnCase("t936_h16x32", 16, 32, [936], seed=9),
    "t3399_h16x32": GdnCase("t3399_h16x32", 16, 32, [3399], seed=4),
    "t16384_h16x32": GdnCase("t16384_h16x32", 16, 32, [16384], seed=5),
    # one GPU's share of T = 16,384 when the 32 v-heads are split over 8 GPUs by heads
    "t16384_h2x4": GdnCase("t16384_h2x4", 2, 4, [16384], seed=6),
}


@dataclass
class GdnInputs:
    q: np.ndarray        # uint16 bf16 bits [T, Hk, D]
    k: np.ndarray        # uint16 bf16 bits [T, Hk, D]
    v: np.ndarray        # uint16 bf16 bits [T, Hv, D]
    beta: np.ndarray     # float32 [T, Hv]
    g: np.ndarray        # float32 [T, Hv]
    cu: np.ndarray       # int32 [N+1]
    h0: Optional[np.ndarray] = None  # float32 [N, Hv, D, D] (key-major) or None
    extra: dict = field(default_factory=dict)

    def f64(self):
        """fp64 views of exactly the stored values (what the oracle consumes)."""
        return (bits_to_f64(self.q), bits_to_f64(self.k), bits_to_f64(self.v),
                self.g.astype(np.float64), self.beta.astype(np.float64), self.cu.astype(np.int64),
                None if self.h0 is None else self.h0.astype(np.float64))


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_gdn_inputs(Hk: int, Hv: int, lengths, seed: int, with_h0: bool = False, h0_std: float = 0.05,
                    g_mean: float = 3.0, d: int = D) -> GdnInputs:
    """Draw q, k, v, beta, g (and h0) in this order from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    q = bf16_bits(_unit_rows(rng.standard_normal((T, Hk, d))))
    k = bf16_bits(_unit_rows(rng.standard_normal((T, Hk, d))))
    v = bf16_bits(rng.standard_normal((T, Hv, d)))
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))).astype(np.float32)
    x = g_mean + rng.standard_normal((T, Hv))
    g = (-np.log1p(np.exp(-x))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32) if lengths else np.zeros(1, np.int32)
    h0 = None
    if with_h0:
        h0 = (h0_std * rng.standard_normal((len(lengths), Hv, d, d))).astype(np.float32)
    return GdnInputs(q, k, v, beta, g, cu, h0)


def make_case(name: str) -> GdnInputs:
    c = CASES[name]
    return make_gdn_inputs(c.Hk, c.Hv, c.lengths, c.seed, c.with_h0, c.h0_std, c.g_mean)


# ----------------------------------------------------------------------------------------------
# Mixer inputs: one GDN layer at T=936, Hk=16, Hv=32, d=128; layer l uses seed 100 + l.
# ----------------------------------------------------------------------------------------------
MIXER_T = 936
MIXER_LAYERS = 48


@dataclass
class MixerInputs:
    qkv: np.ndarray      # uint16 bf16 bits [T, 2*Hk*D + Hv*D]
    conv_w: np.ndarray   # uint16 bf16 bits [2*Hk*D + Hv*D, 4]
    beta: np.ndarray     # float32 [T, Hv]
    g: np.ndarray        # float32 [T, Hv]
    z: np.ndarray        # uint16 bf16 bits [T, Hv, D]
    norm_w: np.ndarray   # uint16 bf16 bits [D]
    cu: np.ndarray       # int32 [N+1]
    h0: Optional[np.ndarray] = None


def make_mixer_inputs(seed: int, lengths=(MIXER_T,), Hk: int = 16, Hv: int = 32, d: int = D,
                      with_h0: bool = False) -> MixerInputs:
    """qkv ~ N(0,1), conv_w ~ 0.5 N(0,1), beta, g as above, z ~ N(0,1), norm_w = 1 + 0.1 N(0,1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    C = 2 * Hk * d + Hv * d
    qkv = bf16_bits(rng.standard_normal((T, C)))
    conv_w = bf16_bits(0.5 * rng.standard_normal((C, 4)))
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))).astype(np.float32)
    x = 3.0 + rng.standard_normal((T, Hv))
    g = (-np.log1p(np.exp(-x))).astype(np.float32)
    z = bf16_bits(rng.standard_normal((T, Hv, d)))
    norm_w = bf16_bits(1.0 + 0.1 * rng.standard_normal(d))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    h0 = (0.05 * rng.standard_normal((len(lengths), Hv, d, d))).astype(np.float32) if with_h0 else None
    return MixerInputs(qkv, conv_w, beta, g, z, norm_w, cu, h0)


@dataclass
class GateInputs:
    a: np.ndarray        # uint16 bf16 bits [T, Hv]: the projection row that sets the decay
    b: np.ndarray        # uint16 bf16 bits [T, Hv]: the projection row that sets beta
    A_log: np.ndarray    # float32 [Hv]
    dt_bias: np.ndarray  # float32 [Hv]


def make_gate_inputs(seed: int, T: int, Hv: int) -> GateInputs:
    """Inputs of the gate-parameter step: a, b ~ N(0, 1) in bf16; per head A_log = log A with
    A ~ U(1, 16) and dt_bias = log(expm1(dt)) with log dt ~ U(log 1e-3, log 1e-1), the customary
    initialisation of a Mamba2-style gate (softplus(dt_bias) = dt)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = bf16_bits(rng.standard_normal((T, Hv)))
    b = bf16_bits(rng.standard_normal((T, Hv)))
    A_log = np.log(rng.uniform(1.0, 16.0, Hv)).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), Hv))
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    return GateInputs(a, b, A_log, dt_bias)


# ----------------------------------------------------------------------------------------------
# Carried states for continuation: pools of initial recurrent states and conv input windows.
# ----------------------------------------------------------------------------------------------
def make_state_pool(seed: int, S: int, Hv: int, d: int = D, std: float = 0.05) -> np.ndarray:
    """S initial states, fp32 [S, Hv, d, d] ~ std N(0,1) (key-major, as h0)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (std * rng.standard_normal((S, Hv, d, d))).astype(np.float32)


def make_window_pool(seed: int, S: int, C: int, taps: int = 4) -> np.ndarray:
    """S conv input windows, bf16 bits [S, taps-1, C] ~ N(0,1) (qkv rows, oldest first)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits(rng.standard_normal((S, taps - 1, C)))

