"""Pins for the retention (decayed / gated linear attention) oracle, against
what the page and the mathematics fix.

Source: "08 - Transformer and Variants" (by-xin.github.io), section 1.3.4:
H_t = gamma_t H_{t-1} + v_t k_t^T, y_t = H_t q_t (RetNet: constant gamma;
gated retention: gamma_t per token); section 1.3.1: with gamma = 1 the state
is the plain sum D_1 + ... + D_t.
"""

import math
import os
import types

import numpy as np
import pytest

import oracle
from oracle import retention_oracle as ret
from workloads import numpy_inputs, rel_l2


def gates(shape, seed, lo=0.6, hi=1.0):
    """log gamma for gamma ~ U(lo, hi)."""
    return np.log(np.random.default_rng(seed).uniform(lo, hi, shape))


def test_hand_example_constant_decay():
    # D = M = 1, gamma = 1/2: y_1 = q1 k1 v1, y_2 = q2 (k1 v1 / 2 + k2 v2),
    # y_3 = q3 (k1 v1 / 4 + k2 v2 / 2 + k3 v3)
    q = np.array([[2.0], [-1.0], [3.0]])
    k = np.array([[1.0], [4.0], [-2.0]])
    v = np.array([[5.0], [1.0], [0.5]])
    lg = np.full(3, math.log(0.5))
    want = np.array([[10.0], [-(2.5 + 4.0)], [3.0 * (1.25 + 2.0 - 1.0)]])
    for y in (ret.recurrent(q, k, v, lg)[0], ret.quadratic(q, k, v, lg)):
        np.testing.assert_allclose(y, want, rtol=1e-14)


def test_constant_inputs_closed_form():
    # q = k = v = 1 (D = M = 1): y_t = sum_{j <= t} gamma^{t-j} = (1 - gamma^{t+1}) / (1 - gamma)
    n, gam = 40, 0.9
    ones = np.ones((n, 1))
    y = ret.quadratic(ones, ones, ones, np.full(n, math.log(gam)))
    t = np.arange(n)
    np.testing.assert_allclose(y[:, 0], (1 - gam ** (t + 1)) / (1 - gam), rtol=1e-12)


def test_long_strongly_gated_sequence_stays_finite():
    # cumulative log decay far below the exponent range: only the current
    # and the few latest tokens matter, and the masked sum must not overflow
    q, k, v, _ = numpy_inputs(1, 1, 3000, 3, 2, seed=66, scale=1.0)
    lg = np.full((1, 1, 3000), math.log(0.05))
    y = ret.quadratic(q, k, v, lg)
    assert np.isfinite(y).all()
    np.testing.assert_allclose(y, ret.recurrent(q, k, v, lg)[0], rtol=1e-10, atol=1e-12)


def test_zero_decay_keeps_only_the_current_token():
    q, k, v, _ = numpy_inputs(1, 2, 9, 4, 3, seed=51, scale=1.0)
    y = ret.recurrent(q, k, v, np.full((1, 2, 9), -800.0))[0]
    want = (q * k).sum(-1)[..., None] * v
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("with_state", [False, True])
def test_two_forms_agree(with_state):
    q, k, v, _ = numpy_inputs(2, 3, 17, 5, 4, seed=52, scale=1.0)
    lg = gates((2, 3, 17), 53)
    S0 = np.random.default_rng(54).standard_normal((2, 3, 5, 4)) if with_state else None
    np.testing.assert_allclose(ret.recurrent(q, k, v, lg, S0)[0], ret.quadratic(q, k, v, lg, S0), rtol=1e-11,
                               atol=1e-12)


def test_bruteforce_scalar_loops():
    q, k, v, _ = numpy_inputs(1, 1, 7, 3, 2, seed=55, scale=1.0)
    lg = gates((1, 1, 7), 56)
    np.testing.assert_allclose(ret.quadratic(q, k, v, lg)[0, 0], ret.bruteforce(q[0, 0], k[0, 0], v[0, 0], lg[0, 0]),
                               rtol=1e-12)


def test_no_decay_is_the_linear_attention_numerator():
    # gamma = 1 on phi(q), phi(k): y_i = phi(Q_i)^T S_i, the numerator of the
    # linear-attention readout (out * den of that oracle)
    q, k, v, _ = numpy_inputs(2, 2, 12, 4, 3, seed=57, scale=1.0)
    y = ret.recurrent(oracle.phi(q), oracle.phi(k), v, np.zeros((2, 2, 12)))[0]
    out, den = oracle.forward_recurrent(q, k, v, True)[:2]
    np.testing.assert_allclose(y, out * den[..., None], rtol=1e-12)


def test_state_continues_the_sequence_and_decode_steps():
    q, k, v, _ = numpy_inputs(1, 2, 15, 4, 3, seed=58, scale=1.0)
    lg = gates((1, 2, 15), 59)
    full, S_full = ret.recurrent(q, k, v, lg)
    a = 6
    _, Sa = ret.recurrent(q[..., :a, :], k[..., :a, :], v[..., :a, :], lg[..., :a])
    rest = ret.quadratic(q[..., a:, :], k[..., a:, :], v[..., a:, :], lg[..., a:], Sa)
    np.testing.assert_allclose(rest, full[..., a:, :], rtol=1e-11, atol=1e-12)
    S = np.zeros((1, 2, 4, 3))
    for t in range(15):
        S, yt = ret.decode_step(S, q[..., t, :], k[..., t, :], v[..., t, :], lg[..., t])
        np.testing.assert_allclose(yt, full[..., t, :], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, S_full, rtol=1e-12)


@pytest.mark.parametrize("with_state", [False, True])
def test_backward_matches_finite_differences(with_state):
    q, k, v, g = numpy_inputs(1, 1, 6, 3, 2, seed=60, scale=1.0)
    lg = gates((1, 1, 6), 61)
    S0 = np.random.default_rng(62).standard_normal((1, 1, 3, 2)) if with_state else None
    got = ret.backward(q, k, v, lg, g, S0)
    fd = ret.fd_grad(q, k, v, lg, g, S0)
    for a, b in zip(got, fd):
        assert rel_l2(a, b) < 1e-6
    if not with_state:
        # dS0 is still defined (the state that would have been carried in)
        fd_s = ret.fd_grad(q, k, v, lg, g, np.zeros((1, 1, 3, 2)))[4]
        assert rel_l2(got[4], fd_s) < 1e-6


# ---------------------------------------------------------- mutants -------
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "retention_oracle.py")


def load_variant(old, new):
    text = open(SRC).read()
    assert old in text, old
    mod = types.ModuleType("retention_mutant")
    exec(compile(text.replace(old, new), "retention_mutant", "exec"), mod.__dict__)
    return mod


def pins_pass(o) -> bool:
    q = np.array([[2.0], [-1.0], [3.0]])
    k = np.array([[1.0], [4.0], [-2.0]])
    v = np.array([[5.0], [1.0], [0.5]])
    want = np.array([[10.0], [-6.5], [6.75]])
    lg3 = np.full(3, math.log(0.5))
    if not (np.allclose(o.recurrent(q, k, v, lg3)[0], want) and np.allclose(o.quadratic(q, k, v, lg3), want)):
        return False
    q, k, v, g = numpy_inputs(1, 1, 6, 3, 2, seed=63, scale=1.0)
    lg = gates((1, 1, 6), 64)
    S0 = np.random.default_rng(65).standard_normal((1, 1, 3, 2))
    if not np.allclose(o.recurrent(q, k, v, lg, S0)[0], o.quadratic(q, k, v, lg, S0), rtol=1e-11):
        return False
    for a, b in zip(o.backward(q, k, v, lg, g, S0), o.fd_grad(q, k, v, lg, g, S0)):
        if not rel_l2(a, b) < 1e-6:
            return False
    return True


RET_MUTANTS = {
    "decay_after_update": (
        "S = np.exp(lg[..., t])[..., None, None] * S + k[..., t, :, None] * v[..., t, None, :]\n        y[",
        "S = np.exp(lg[..., t])[..., None, None] * (S + k[..., t, :, None] * v[..., t, None, :])\n        y["),
    "decay_exponent_sign": ("L[..., :, None] - L[..., None, :], 0.0)", "L[..., None, :] - L[..., :, None], 0.0)"),
    "state_not_decayed_in_quadratic": ("y = y + np.exp(L)[..., None] * (q @ _f64(S0))", "y = y + (q @ _f64(S0))"),
    "forward_cumsum_for_gates": ("dlg = np.flip(np.cumsum(np.flip(per_token, -1), -1), -1)",
                                 "dlg = np.cumsum(per_token, -1)"),
    "suffix_state_decayed_by_wrong_gate": ("R = np.exp(lg[..., t + 1])[..., None, None] * R",
                                           "R = np.exp(lg[..., t])[..., None, None] * R"),
    "dS0_misses_first_gate": ("dS0 = np.exp(lg[..., 0])[..., None, None] * R", "dS0 = R"),
}


def test_unmodified_retention_copy_passes():
    assert pins_pass(load_variant("import math", "import math"))


@pytest.mark.parametrize("name", sorted(RET_MUTANTS))
def test_retention_mutant_is_caught(name):
    assert not pins_pass(load_variant(*RET_MUTANTS[name])), name
