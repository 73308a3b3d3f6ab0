"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, never against the oracle's own formulas retyped.

Sources (page title, section / equation):
* "[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io): section 2
  (phi = elu + 1), section 3 (eq:mask, the S_i / Z_i recurrence, eq:output),
  section 3.1 (eq:gq .. eq:gv), section 4 (the RNN form).
* "The deep link between Transformer and RNN" (xxqk.cn), section 3 (decode
  loop: update, then read).
"""

import math

import numpy as np
import pytest

import oracle
from workloads import numpy_inputs, rel_l2


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- phi -----
def test_phi_closed_form():
    # elu(x) + 1 with alpha = 1: x + 1 above zero, e^x at or below zero.
    x = np.array([0.0, 1.0, -1.0, 2.5, -3.0, 1e-300, -1e-300, -800.0])
    want = np.array([1.0, 2.0, math.exp(-1.0), 3.5, math.exp(-3.0), 1.0, 1.0, 0.0])
    np.testing.assert_allclose(oracle.phi(x), want, rtol=0, atol=1e-15)
    assert np.all(oracle.phi(rand(1000, 1, 5.0)) > 0)


def test_phi_prime_matches_central_difference():
    x = np.concatenate([rand(200, 2, 3.0), [0.5, -0.5, 1e-3, -1e-3]])
    h = 1e-6
    fd = (oracle.phi(x + h) - oracle.phi(x - h)) / (2 * h)
    np.testing.assert_allclose(oracle.phi_prime(x), fd, rtol=1e-8, atol=1e-9)
    # phi is C^1 at zero: both one-sided slopes are 1.
    assert oracle.phi_prime(np.array([0.0]))[0] == 1.0
    assert abs((oracle.phi(1e-7) - oracle.phi(0.0)) / 1e-7 - 1.0) < 1e-6
    assert abs((oracle.phi(0.0) - oracle.phi(-1e-7)) / 1e-7 - 1.0) < 1e-6


# ------------------------------------------------------------ forward -----
def test_hand_worked_example_d1():
    # D = M = 1: phi(q) cancels between numerator and denominator, so row i
    # is the phi(k)-weighted mean of v_1..v_i.  phi(0) = 1, phi(1) = 2,
    # phi(-1) = 1/e (closed form, no library call of the oracle's).
    q = np.array([[0.3], [-2.0], [1.7]])
    k = np.array([[0.0], [1.0], [-1.0]])
    v = np.array([[3.0], [6.0], [9.0]])
    e1 = math.exp(-1.0)
    want = np.array([[3.0], [(3.0 + 2 * 6.0) / 3.0], [(3.0 + 12.0 + 9.0 * e1) / (3.0 + e1)]])
    for fn in (lambda: oracle.forward_quadratic(q, k, v, True)[0],
               lambda: oracle.forward_recurrent(q, k, v, True)[0],
               lambda: oracle.forward_bruteforce(q, k, v, True)):
        np.testing.assert_allclose(fn(), want, rtol=1e-15)
    # Non-causal: every row is the last causal row.
    nc = oracle.forward_quadratic(q, k, v, False)[0]
    np.testing.assert_allclose(nc, np.repeat(want[-1:], 3, axis=0), rtol=1e-15)
    # den_i = phi(q_i) * Z_i with Z = cumulative phi(k) = 1, 3, 3 + 1/e.
    den = oracle.forward_recurrent(q, k, v, True)[1]
    phq = np.array([1.3, math.exp(-2.0), 2.7])
    np.testing.assert_allclose(den, phq * np.array([1.0, 3.0, 3.0 + e1]), rtol=1e-15)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 1, 1, 4, 4), (2, 3, 17, 5, 7), (1, 2, 70, 16, 16), (1, 1, 33, 8, 3)])
def test_quadratic_equals_recurrence(causal, shape):
    B, H, N, D, M = shape
    q, k, v, _ = numpy_inputs(B, H, N, D, M, seed=N, scale=1.0)
    oq, dq_ = oracle.forward_quadratic(q, k, v, causal)
    orr, dr, _, _ = oracle.forward_recurrent(q, k, v, causal)
    assert rel_l2(orr, oq) < 1e-12
    assert rel_l2(dr, dq_) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_bruteforce_scalar_loops(causal):
    q, k, v = rand((6, 3), 10), rand((6, 3), 11), rand((6, 2), 12)
    ob = oracle.forward_bruteforce(q, k, v, causal)
    oq = oracle.forward_quadratic(q, k, v, causal)[0]
    np.testing.assert_allclose(oq, ob, rtol=1e-13, atol=1e-14)


def test_single_token_returns_v():
    q, k, v = rand((3, 1, 8), 1), rand((3, 1, 8), 2), rand((3, 1, 5), 3)
    for causal in (True, False):
        np.testing.assert_allclose(oracle.forward_quadratic(q, k, v, causal)[0], v, rtol=1e-15)
        np.testing.assert_allclose(oracle.forward_recurrent(q, k, v, causal)[0], v, rtol=1e-15)


def test_zero_keys_give_running_mean():
    # K = 0 => phi(K) = 1 => every key weighs the same => textbook running mean.
    n = 50
    q, v = rand((n, 6), 4), rand((n, 4), 5)
    k = np.zeros((n, 6))
    mean = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(oracle.forward_recurrent(q, k, v, True)[0], mean, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.forward_quadratic(q, k, v, True)[0], mean, rtol=1e-13, atol=1e-15)
    gm = np.broadcast_to(v.mean(axis=0), v.shape)
    np.testing.assert_allclose(oracle.forward_quadratic(q, k, v, False)[0], gm, rtol=1e-13, atol=1e-15)


def test_d1_output_independent_of_q():
    k, v = rand((30, 1), 6), rand((30, 3), 7)
    a = oracle.forward_recurrent(rand((30, 1), 8), k, v, True)[0]
    b = oracle.forward_recurrent(rand((30, 1), 9, 4.0), k, v, True)[0]
    np.testing.assert_allclose(a, b, rtol=1e-13)


def test_affine_equivariance_and_convex_hull():
    q, k, v = rand((2, 40, 8), 13), rand((2, 40, 8), 14), rand((2, 40, 5), 15)
    a, b = 2.5, rand(5, 16)
    base = oracle.forward_recurrent(q, k, v, True)[0]
    moved = oracle.forward_recurrent(q, k, a * v + b, True)[0]
    np.testing.assert_allclose(moved, a * base + b, rtol=1e-12, atol=1e-12)
    lo = np.minimum.accumulate(v, axis=-2)
    hi = np.maximum.accumulate(v, axis=-2)
    assert np.all(base >= lo - 1e-12) and np.all(base <= hi + 1e-12)


def test_noncausal_rows_read_final_state():
    q, k, v = rand((1, 2, 25, 6), 17), rand((1, 2, 25, 6), 18), rand((1, 2, 25, 4), 19)
    oc = oracle.forward_quadratic(q, k, v, True)[0]
    onc = oracle.forward_quadratic(q, k, v, False)[0]
    np.testing.assert_allclose(onc[..., -1, :], oc[..., -1, :], rtol=1e-13)
    # Every non-causal row is the causal readout of its query against the
    # final state: append query i after the sequence as a decode step whose
    # key weighs nothing is not expressible, so instead place query i at the
    # last position of a causal run over the same keys and values.
    for i in (0, 7, 24):
        q2 = q.copy()
        q2[..., -1, :] = q[..., i, :]
        last = oracle.forward_quadratic(q2, k, v, True)[0][..., -1, :]
        np.testing.assert_allclose(onc[..., i, :], last, rtol=1e-12)
    S, Z = oracle.prefix_state(k, v)
    _, _, S2, Z2 = oracle.forward_recurrent(q, k, v, False)
    np.testing.assert_allclose(S, S2, rtol=1e-13)
    np.testing.assert_allclose(Z, Z2, rtol=1e-13)


# ------------------------------------------------------------- decode -----
def test_decode_equals_parallel_form():
    # RNN form from s_0 = z_0 = 0 reproduces the causal rows.
    B, H, N, D, M = 2, 3, 20, 8, 6
    q, k, v, _ = numpy_inputs(B, H, N, D, M, seed=21, scale=1.0)
    S = np.zeros((B, H, D, M))
    Z = np.zeros((B, H, D))
    qs, ks, vs = (np.moveaxis(x, 2, 0) for x in (q, k, v))
    S, Z, outs = oracle.decode_steps(S, Z, qs, ks, vs)
    par = oracle.forward_quadratic(q, k, v, True)[0]
    np.testing.assert_allclose(np.moveaxis(outs, 0, 2), par, rtol=1e-12)
    S2, Z2 = oracle.prefix_state(k, v)
    np.testing.assert_allclose(S, S2, rtol=1e-12)
    np.testing.assert_allclose(Z, Z2, rtol=1e-12)


def test_decode_from_prefix_state():
    B, H, P, T, D, M = 1, 2, 12, 9, 5, 4
    q, k, v, _ = numpy_inputs(B, H, P + T, D, M, seed=22, scale=1.0)
    S, Z = oracle.prefix_state(k[..., :P, :], v[..., :P, :])
    qs, ks, vs = (np.moveaxis(x[..., P:, :], 2, 0) for x in (q, k, v))
    _, _, outs = oracle.decode_steps(S, Z, qs, ks, vs)
    par = oracle.forward_quadratic(q, k, v, True)[0][..., P:, :]
    np.testing.assert_allclose(np.moveaxis(outs, 0, 2), par, rtol=1e-12)
    # state carried into the recurrence gives the same rows
    rec = oracle.forward_recurrent(q[..., P:, :], k[..., P:, :], v[..., P:, :], True, S, Z)[0]
    np.testing.assert_allclose(rec, par, rtol=1e-12)


# ----------------------------------------------------------- backward -----
@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_finite_differences_tiny(causal):
    # The tiny workload's shape: B=H=1, N=64, D=M=16, unscaled N(0,1), seed 0.
    q, k, v, g = numpy_inputs(1, 1, 64, 16, 16, seed=0, scale=1.0)
    dq, dk, dv, _, _ = oracle.backward(q, k, v, g, causal)
    fq, fk, fv = oracle.fd_grad(q, k, v, g, causal)
    assert rel_l2(dq, fq) < 1e-6
    assert rel_l2(dk, fk) < 1e-6
    assert rel_l2(dv, fv) < 1e-6


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_finite_differences_rect(causal):
    q, k, v, g = numpy_inputs(2, 1, 11, 3, 5, seed=3, scale=1.0)
    dq, dk, dv, _, _ = oracle.backward(q, k, v, g, causal)
    fq, fk, fv = oracle.fd_grad(q, k, v, g, causal)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        assert rel_l2(a, b) < 1e-6


@pytest.mark.parametrize("causal", [True, False])
def test_backward_dv_sums_to_dout_sum(causal):
    # each output row's weights sum to one, so sum_j dV_j = sum_i G_i
    q, k, v, g = numpy_inputs(2, 2, 30, 6, 4, seed=5, scale=1.0)
    dv = oracle.backward(q, k, v, g, causal)[2]
    np.testing.assert_allclose(dv.sum(axis=-2), g.sum(axis=-2), rtol=1e-12, atol=1e-12)


def test_backward_zero_keys_give_zero_dq():
    q, _, v, g = numpy_inputs(1, 1, 20, 4, 3, seed=6, scale=1.0)
    k = np.zeros_like(q)
    for causal in (True, False):
        dq = oracle.backward(q, k, v, g, causal)[0]
        assert np.max(np.abs(dq)) < 1e-14


def test_backward_returns_forward_output():
    q, k, v, g = numpy_inputs(1, 2, 15, 4, 4, seed=7, scale=1.0)
    out, den = oracle.backward(q, k, v, g, True)[3:]
    oq, dq_ = oracle.forward_quadratic(q, k, v, True)
    np.testing.assert_allclose(out, oq, rtol=1e-12)
    np.testing.assert_allclose(den, dq_, rtol=1e-12)


# ------------------------------------------------------ frozen snapshot ---
# ------------------------------------------------- carried-in state -----
# A state (S0, Z0) from earlier tokens: the walkthrough's section 4 starts
# the recurrence from s_0 = z_0 = 0, and "The deep link between Transformer
# and RNN" (xxqk.cn), section 4.2, saves and restores a session's state.
# Carrying the state of a prefix must reproduce the plain definition over the
# concatenated tokens.
@pytest.mark.parametrize("causal", [True, False])
def test_state_forms_agree(causal):
    q, k, v, _ = numpy_inputs(2, 2, 9, 3, 4, seed=31, scale=1.0)
    S0 = rand((2, 2, 3, 4), 32)
    Z0 = np.abs(rand((2, 2, 3), 33)) + 0.5  # a valid Z is positive
    o1, d1 = oracle.forward_quadratic(q, k, v, causal, S0, Z0)
    o2, d2, S2, Z2 = oracle.forward_recurrent(q, k, v, causal, S0, Z0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12)
    np.testing.assert_allclose(d1, d2, rtol=1e-12)
    Sp, Zp = oracle.prefix_state(k, v)
    np.testing.assert_allclose(S2, S0 + Sp, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Z2, Z0 + Zp, rtol=1e-12)


def test_state_of_prefix_continues_the_sequence():
    # rows a..N of the causal definition over N tokens == the rows computed
    # over tokens a..N alone, starting from the state of tokens 0..a-1
    q, k, v, _ = numpy_inputs(1, 2, 13, 4, 3, seed=34, scale=1.0)
    full, dfull = oracle.forward_quadratic(q, k, v, True)
    for a in (1, 5, 12):
        S0, Z0 = oracle.prefix_state(k[..., :a, :], v[..., :a, :])
        part, dpart = oracle.forward_quadratic(q[..., a:, :], k[..., a:, :], v[..., a:, :], True, S0, Z0)
        np.testing.assert_allclose(part, full[..., a:, :], rtol=1e-12)
        np.testing.assert_allclose(dpart, dfull[..., a:], rtol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_state_matches_finite_differences(causal):
    q, k, v, g = numpy_inputs(1, 1, 6, 3, 2, seed=35, scale=1.0)
    S0 = rand((1, 1, 3, 2), 36)
    Z0 = np.abs(rand((1, 1, 3), 37)) + 0.5
    dq, dk, dv, dS0, dZ0, _, _ = oracle.backward_state(q, k, v, g, S0, Z0, causal)
    fq, fk, fv, fS, fZ = oracle.fd_grad_state(q, k, v, g, S0, Z0, causal)
    for a, b in ((dq, fq), (dk, fk), (dv, fv), (dS0, fS), (dZ0, fZ)):
        assert rel_l2(a, b) < 1e-6


def test_state_gradients_are_what_the_prefix_tokens_receive():
    # Over [prefix | rest] with dout = 0 on the prefix rows, a prefix token's
    # value and key reach the loss only through the rest's state S0, Z0, so
    # dv_p = dS0^T phi(K_p) and grad phi(K_p) = dS0 v_p + dZ0.
    q, k, v, g = numpy_inputs(1, 2, 11, 3, 4, seed=38, scale=1.0)
    a = 4
    g = g.copy()
    g[..., :a, :] = 0.0
    dq, dk, dv, _, _ = oracle.backward(q, k, v, g, True)
    S0, Z0 = oracle.prefix_state(k[..., :a, :], v[..., :a, :])
    rest = (x[..., a:, :] for x in (q, k, v, g))
    rq, rk, rv, dS0, dZ0, _, _ = oracle.backward_state(*rest, S0, Z0, True)
    np.testing.assert_allclose(rq, dq[..., a:, :], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(rk, dk[..., a:, :], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(rv, dv[..., a:, :], rtol=1e-10, atol=1e-14)
    kf = oracle.phi(k[..., :a, :])
    np.testing.assert_allclose(dv[..., :a, :], np.einsum("...dm,...pd->...pm", dS0, kf), rtol=1e-10)
    dkf = np.einsum("...dm,...pm->...pd", dS0, v[..., :a, :]) + dZ0[..., None, :]
    np.testing.assert_allclose(dk[..., :a, :], dkf * oracle.phi_prime(k[..., :a, :]), rtol=1e-10)


def test_backward_state_zero_state_is_backward():
    q, k, v, g = numpy_inputs(1, 2, 8, 3, 3, seed=39, scale=1.0)
    for causal in (True, False):
        a = oracle.backward(q, k, v, g, causal)
        b = oracle.backward_state(q, k, v, g, np.zeros((1, 2, 3, 3)), np.zeros((1, 2, 3)), causal)
        for x, y in zip(a[:3], b[:3]):
            np.testing.assert_allclose(x, y, rtol=1e-13)


def test_oracle_matches_frozen_snapshot():
    # tests/golden/oracle_small.json was written by tests/golden/make_golden.py
    # (oracle only); a change here means the oracle's arithmetic changed.
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")
    rec = json.load(open(path))
    B, H, N, D, M = rec["shape"]
    q, k, v, g = numpy_inputs(B, H, N, D, M, seed=rec["seed"], scale=rec["scale"])
    for causal in (True, False):
        want = rec["causal" if causal else "noncausal"]
        out, den = oracle.forward_quadratic(q, k, v, causal)
        dq, dk, dv, _, _ = oracle.backward(q, k, v, g, causal)
        for name, got in (("out", out), ("den", den), ("dq", dq), ("dk", dk), ("dv", dv)):
            np.testing.assert_allclose(got, np.array(want[name]), rtol=1e-12, atol=1e-14)
