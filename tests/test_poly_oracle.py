"""Pins for the degree-2 polynomial-kernel oracle, against what the page and
the mathematics fix.

Source: "[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io),
section 2, "feature map and computation cost", item (3): (x^T y)^2 =
sum_i sum_j (x_i x_j)(y_i y_j), C = D^2; the attention is ``eq:common`` with
that kernel, causal per ``eq:mask``.
"""

import os
import types

import numpy as np
import pytest

from oracle import poly_oracle as po
from workloads import numpy_inputs, rel_l2


def test_feature_identity_hand_example():
    # x = [1, 2], y = [3, -1]: x.y = 1; phi(x) = [1, 2, 2, 4], phi(y) = [9, -3, -3, 1]
    x, y = np.array([1.0, 2.0]), np.array([3.0, -1.0])
    np.testing.assert_array_equal(po.phi2(x), [1.0, 2.0, 2.0, 4.0])
    np.testing.assert_array_equal(po.phi2(y), [9.0, -3.0, -3.0, 1.0])
    assert po.phi2(x) @ po.phi2(y) == 1.0


def test_feature_identity_random():
    rng = np.random.default_rng(1)
    x, y = rng.standard_normal((2, 50, 7))
    scale = ((x * x).sum(-1) * (y * y).sum(-1)).max()
    np.testing.assert_allclose((po.phi2(x) * po.phi2(y)).sum(-1), (x * y).sum(-1) ** 2, rtol=1e-12, atol=1e-13 * scale)


def test_hand_example_one_feature():
    # D = M = 1, q = 1: weights k_j^2 -> out = running weighted means
    q = np.ones((3, 1))
    k = np.array([[1.0], [2.0], [-1.0]])
    v = np.array([[1.0], [2.0], [3.0]])
    want = np.array([[1.0], [9.0 / 5.0], [12.0 / 6.0]])
    out, den = po.forward_quadratic(q, k, v)
    np.testing.assert_allclose(out, want, rtol=1e-15)
    np.testing.assert_allclose(den, [1.0, 5.0, 6.0])
    np.testing.assert_allclose(po.forward_recurrent(q, k, v)[0], want, rtol=1e-15)
    np.testing.assert_allclose(po.forward_bruteforce(q, k, v), want, rtol=1e-15)
    # non-causal: every row is the full weighted mean 12 / 6
    np.testing.assert_allclose(po.forward_quadratic(q, k, v, causal=False)[0], np.full((3, 1), 2.0))


@pytest.mark.parametrize("causal", [True, False])
def test_two_forms_agree(causal):
    q, k, v, _ = numpy_inputs(2, 3, 13, 4, 5, seed=2, scale=1.0)
    a = po.forward_quadratic(q, k, v, causal)
    b = po.forward_recurrent(q, k, v, causal)
    np.testing.assert_allclose(b[0], a[0], rtol=1e-11)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-11)


@pytest.mark.parametrize("causal", [True, False])
def test_bruteforce(causal):
    q, k, v, _ = numpy_inputs(1, 1, 9, 3, 2, seed=3, scale=1.0)
    np.testing.assert_allclose(po.forward_quadratic(q, k, v, causal)[0][0, 0],
                               po.forward_bruteforce(q[0, 0], k[0, 0], v[0, 0], causal), rtol=1e-12)


def test_zero_denominator_reads_zero():
    # q_0 = 0: every weight of row 0 vanishes; q_1 orthogonal to both keys
    q = np.array([[0.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    k = np.array([[1.0, 0.0], [2.0, 0.0], [1.0, 3.0]])
    v = np.array([[5.0], [7.0], [1.0]])
    out, den = po.forward_quadratic(q, k, v)
    assert den[0] == 0 and den[1] == 0 and den[2] > 0
    np.testing.assert_array_equal(out[:2], 0.0)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(po.forward_recurrent(q, k, v)[0], out, rtol=1e-15)
    np.testing.assert_allclose(po.forward_bruteforce(q, k, v), out, rtol=1e-15)


def test_sign_and_scale_invariance():
    # the weights are homogeneous of degree 2 in q and in k, and even
    q, k, v, _ = numpy_inputs(1, 2, 11, 4, 3, seed=4, scale=1.0)
    base = po.forward_quadratic(q, k, v)[0]
    for qq, kk in ((-q, k), (q, -k), (3.0 * q, k), (q, 0.25 * k), (-2.0 * q, -5.0 * k)):
        np.testing.assert_allclose(po.forward_quadratic(qq, kk, v)[0], base, rtol=1e-12)


def test_state_continues_the_sequence_and_decode_steps():
    q, k, v, _ = numpy_inputs(1, 2, 14, 3, 4, seed=5, scale=1.0)
    full = po.forward_quadratic(q, k, v)[0]
    a = 5
    S, Z = po.prefix_state(k[..., :a, :], v[..., :a, :])
    rest = po.forward_recurrent(q[..., a:, :], k[..., a:, :], v[..., a:, :], True, S, Z)[0]
    np.testing.assert_allclose(rest, full[..., a:, :], rtol=1e-11)
    for t in range(a, 14):
        S, Z, o = po.decode_step(S, Z, q[..., t, :], k[..., t, :], v[..., t, :])
        np.testing.assert_allclose(o, full[..., t, :], rtol=1e-11)
    Sf, Zf = po.prefix_state(k, v)
    np.testing.assert_allclose(S, Sf, rtol=1e-12)
    np.testing.assert_allclose(Z, Zf, rtol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dm", [(3, 3), (2, 4)])
def test_backward_matches_finite_differences(causal, dm):
    D, M = dm
    q, k, v, g = numpy_inputs(1, 1, 6, D, M, seed=6 + D, scale=1.0)
    got = po.backward(q, k, v, g, causal)[:3]
    for a, b in zip(got, po.fd_grad(q, k, v, g, causal)):
        assert rel_l2(a, b) < 1e-6


def test_backward_closed_forms():
    # out is invariant to scaling q_i (each row) and to scaling all keys:
    # q_i . dq_i = 0 for every row and sum_j k_j . dk_j = 0; the weights of a
    # row sum to den_i, so sum_j dv_j = sum_i dout_i
    q, k, v, g = numpy_inputs(2, 2, 17, 5, 3, seed=7, scale=1.0)
    dq, dk, dv, _, _ = po.backward(q, k, v, g)
    scale = np.abs(q * dq).sum(-1).max() + 1e-300
    assert np.abs((q * dq).sum(-1)).max() < 1e-11 * max(1.0, scale)
    assert abs((k * dk).sum()) < 1e-10 * np.abs(k * dk).sum()
    np.testing.assert_allclose(dv.sum(-2), g.sum(-2), rtol=1e-11)


def test_backward_zero_denominator_row_has_no_gradient():
    q = np.array([[0.0, 0.0], [1.0, 0.5], [0.3, -1.0]])
    k = np.array([[1.0, 0.0], [2.0, 1.0], [1.0, 3.0]])
    v = np.array([[5.0], [7.0], [1.0]])
    g = np.array([[1.0], [-2.0], [0.5]])
    dq, dk, dv, _, _ = po.backward(q, k, v, g)
    np.testing.assert_array_equal(dq[0], 0.0)
    for a, b in zip((dq, dk, dv), po.fd_grad(q, k, v, g)):
        assert rel_l2(a, b) < 1e-6


# ---------------------------------------------------------- mutants -------
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "poly_oracle.py")


def load_variant(old, new):
    text = open(SRC).read()
    assert old in text, old
    mod = types.ModuleType("poly_mutant")
    exec(compile(text.replace(old, new), "poly_mutant", "exec"), mod.__dict__)
    return mod


def pins_pass(o) -> bool:
    q = np.ones((3, 1))
    k = np.array([[1.0], [2.0], [-1.0]])
    v = np.array([[1.0], [2.0], [3.0]])
    want = np.array([[1.0], [1.8], [2.0]])
    if not np.allclose(o.forward_quadratic(q, k, v)[0], want):
        return False
    q, k, v, g = numpy_inputs(1, 1, 6, 3, 2, seed=8, scale=1.0)
    if not np.allclose(o.forward_quadratic(q, k, v)[0], o.forward_recurrent(q, k, v)[0], rtol=1e-10):
        return False
    dq, dk, dv, _, _ = o.backward(q, k, v, g)
    for a, b in zip((dq, dk, dv), o.fd_grad(q, k, v, g)):
        if not rel_l2(a, b) < 1e-6:
            return False
    if not np.abs((q * dq).sum(-1)).max() < 1e-10:
        return False
    return bool(np.allclose(dv.sum(-2), g.sum(-2)))


POLY_MUTANTS = {
    "abs_not_square": ("w = (q @ np.swapaxes(k, -1, -2)) ** 2", "w = np.abs(q @ np.swapaxes(k, -1, -2))"),
    "strict_mask": ("w = w * np.tril(np.ones((n, n)))", "w = w * np.tril(np.ones((n, n)), -1)"),
    "no_normaliser": ("return _safe_div(w @ v, den), den", "return w @ v, den"),
    "c_sign": ("c = -(G * out).sum(-1) * inv", "c = (G * out).sum(-1) * inv"),
    "factor_two_dropped": ("ds = 2.0 * s * dw * mask", "ds = s * dw * mask"),
    "dk_untransposed": ("dk = np.swapaxes(ds, -1, -2) @ q", "dk = ds @ q"),
    "dv_unnormalised": ("dv = np.swapaxes(w, -1, -2) @ g", "dv = np.swapaxes(w, -1, -2) @ G"),
    "state_read_before_update": (
        "        Z = Z + fk[..., t, :]\n        num[..., t, :] = np.einsum(\"...c,...cm->...m\", fq[..., t, :], S)",
        "        num[..., t, :] = np.einsum(\"...c,...cm->...m\", fq[..., t, :], S - fk[..., t, :, None] * v[..., t, None, :])\n        Z = Z + fk[..., t, :]"),
}


def test_unmodified_poly_copy_passes():
    assert pins_pass(load_variant("import numpy as np", "import numpy as np"))


@pytest.mark.parametrize("name", sorted(POLY_MUTANTS))
def test_poly_mutant_is_caught(name):
    assert not pins_pass(load_variant(*POLY_MUTANTS[name])), name
