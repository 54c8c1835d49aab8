"""The fp64 oracle against what the mathematics fixes (closed forms, identities, exact rationals,
invariants) and against library routines for the mixer pieces.  CPU only."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.gdn_fwd)


def test_retrieval_full_width():
    # d = 128 with T = 128 orthonormal keys, GQA 16 -> 32 heads shape ratio (Hk=1, Hv=2)
    P.pin_orthonormal_retrieval(oracle.gdn_fwd, d=128, T=128, Hk=1, Hv=2)


def test_chunked_identity_full_width():
    rng = np.random.default_rng(21)
    q, k, v, g, beta, cu, h0 = P._rand_case(rng, 0, 1, 2, 128, lengths=[200, 64, 3], gmean=3.0)
    o, hT = oracle.gdn_fwd(q, k, v, g, beta, cu, h0)
    oc, hc = P.chunked_reference(q, k, v, g, beta, cu, h0)
    assert P._rel(o, oc) < 1e-12 and P._rel(hT, hc) < 1e-12


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(22)
    q, k, v, g, beta, cu, h0 = P._rand_case(rng, 0, 2, 4, 16, lengths=[33, 70])
    a = oracle.gdn_fwd(q, k, v, g, beta, cu, h0, threads=1)
    b = oracle.gdn_fwd(q, k, v, g, beta, cu, h0, threads=8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_zero_length_sequence_keeps_state():
    rng = np.random.default_rng(23)
    q, k, v, g, beta, cu, h0 = P._rand_case(rng, 0, 1, 1, 8, lengths=[0, 5, 0])
    _, hT = oracle.gdn_fwd(q, k, v, g, beta, cu, h0)
    assert np.array_equal(hT[0], h0[0]) and np.array_equal(hT[2], h0[2])


def test_rejects_bad_cu_seqlens():
    z = np.zeros((4, 1, 2))
    with pytest.raises(ValueError):
        oracle.gdn_fwd(z, z, z, np.zeros((4, 1)), np.zeros((4, 1)), [0, 3, 2, 4])


# ---------------------------------------------------------------------------------------------
# Mixer pieces against torch library routines on the CPU in fp64
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("pin", P.MIXER_PINS, ids=lambda f: f.__name__)
def test_mixer_pin(pin):
    pin(oracle.conv_silu, oracle.mixer_fwd, oracle.gdn_fwd)


# ---------------------------------------------------------------------------------------------
# Continuation: states by index, carried conv windows
# ---------------------------------------------------------------------------------------------
def oracle_api(lib=None):
    import functools
    from types import SimpleNamespace
    kw = {} if lib is None else {"lib": lib}
    return SimpleNamespace(fwd=functools.partial(oracle.gdn_fwd, **kw),
                           fwd_idx=functools.partial(oracle.gdn_fwd_indexed, **kw),
                           conv_cont=functools.partial(oracle.conv_silu_cont, **kw),
                           mixer_cont=functools.partial(oracle.mixer_fwd_cont, **kw))


@pytest.mark.parametrize("pin", P.CONT_PINS, ids=lambda f: f.__name__)
def test_continuation_pin(pin):
    pin(oracle_api())


def test_plain_entry_points_equal_the_general_ones():
    # gdn_fwd / mixer_fwd are the indexed / continued forms with identity map and no window
    rng = np.random.default_rng(46)
    q, k, v, g, beta, cu, h0 = P._rand_case(rng, 0, 2, 4, 8, lengths=[10, 3])
    a = oracle.gdn_fwd(q, k, v, g, beta, cu, h0)
    b = oracle.gdn_fwd_indexed(q, k, v, g, beta, cu, h0, [0, 1])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    m = P._mixer_case(rng, [6, 9])
    y, hT = oracle.mixer_fwd(m["qkv"], m["conv_w"], m["g"], m["beta"], m["z"], m["norm_w"], m["cu"],
                             Hk=2, Hv=4, dk=8, dv=8)
    y2, h2, _ = oracle.mixer_fwd_cont(m["qkv"], m["conv_w"], m["g"], m["beta"], m["z"], m["norm_w"], m["cu"],
                                      Hk=2, Hv=4, dk=8, dv=8)
    assert np.array_equal(y, y2) and np.array_equal(hT, h2)


@pytest.mark.parametrize("pin", P.GATE_PINS, ids=lambda f: f.__name__)
def test_gate_pin(pin):
    pin(oracle.gates)
