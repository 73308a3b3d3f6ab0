"""Plant plausible mistakes in a private copy of the oracle (CPU only) and
check that the pins catch each one.  The copy is built from the oracle's
source text with one substitution applied, then loaded as a fresh module;
the real oracle is never modified."""

import math
import os
import types

import numpy as np
import pytest

from workloads import numpy_inputs, rel_l2

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "linattn_oracle.py")


def load_variant(old: str, new: str) -> types.ModuleType:
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor not found: {old!r}"
    text = text.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def pins_pass(o) -> bool:
    """A compact subset of the pins in test_oracle.py; True if all hold."""
    with np.errstate(all="ignore"):
        # hand-worked D = 1 example (closed form)
        q = np.array([[0.3], [-2.0], [1.7]])
        k = np.array([[0.0], [1.0], [-1.0]])
        v = np.array([[3.0], [6.0], [9.0]])
        e1 = math.exp(-1.0)
        want = np.array([[3.0], [5.0], [(15.0 + 9.0 * e1) / (3.0 + e1)]])
        for out in (o.forward_quadratic(q, k, v, True)[0], o.forward_recurrent(q, k, v, True)[0]):
            if not np.allclose(out, want, rtol=1e-13):
                return False
        # brute force, both masks
        qb, kb, vb = (np.random.default_rng(s).standard_normal(sh)
                      for s, sh in ((1, (5, 3)), (2, (5, 3)), (3, (5, 2))))
        for causal in (True, False):
            if not np.allclose(o.forward_quadratic(qb, kb, vb, causal)[0],
                               o.forward_bruteforce(qb, kb, vb, causal), rtol=1e-12):
                return False
        # closed-form backward vs finite differences, D != M, both masks
        q, k, v, g = numpy_inputs(1, 1, 7, 3, 4, seed=9, scale=1.0)
        for causal in (True, False):
            dq, dk, dv, _, _ = o.backward(q, k, v, g, causal)
            fq, fk, fv = o.fd_grad(q, k, v, g, causal)
            for a, b in ((dq, fq), (dk, fk), (dv, fv)):
                if not rel_l2(a, b) < 1e-6:
                    return False
        # decode from zero state vs parallel rows
        q, k, v, _ = numpy_inputs(1, 1, 6, 3, 2, seed=10, scale=1.0)
        S, Z = np.zeros((1, 1, 3, 2)), np.zeros((1, 1, 3))
        _, _, outs = o.decode_steps(S, Z, *(np.moveaxis(x, 2, 0) for x in (q, k, v)))
        if not np.allclose(np.moveaxis(outs, 0, 2), o.forward_quadratic(q, k, v, True)[0], rtol=1e-12):
            return False
        # carried-in state: the rest of a sequence from its prefix's state,
        # and the state gradients vs finite differences
        q, k, v, g = numpy_inputs(1, 1, 7, 3, 2, seed=12, scale=1.0)
        full, _ = o.forward_quadratic(q, k, v, True)
        S0, Z0 = o.prefix_state(k[..., :3, :], v[..., :3, :])
        part, _ = o.forward_recurrent(q[..., 3:, :], k[..., 3:, :], v[..., 3:, :], True, S0, Z0)[:2]
        if not np.allclose(part, full[..., 3:, :], rtol=1e-12):
            return False
        for causal in (True, False):
            got = o.backward_state(q[..., 3:, :], k[..., 3:, :], v[..., 3:, :], g[..., 3:, :], S0, Z0, causal)
            fd = o.fd_grad_state(q[..., 3:, :], k[..., 3:, :], v[..., 3:, :], g[..., 3:, :], S0, Z0, causal)
            for a, b in zip(got[:5], fd):
                if not rel_l2(a, b) < 1e-6:
                    return False
        # prefix state vs the recurrence's final state
        q, k, v, _ = numpy_inputs(1, 1, 6, 3, 2, seed=10, scale=1.0)
        S1, Z1 = o.prefix_state(k, v)
        _, _, S2, Z2 = o.forward_recurrent(q, k, v, False)
        if not (np.allclose(S1, S2, rtol=1e-12) and np.allclose(Z1, Z2, rtol=1e-12)):
            return False
    return True


def test_unmodified_copy_passes():
    assert pins_pass(load_variant("import math", "import math"))


MUTANTS = {
    "relu_plus_one_feature_map": ("np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))",
                                  "np.where(x > 0.0, x + 1.0, 1.0 + 0.0 * x)"),
    "strict_causal_mask": ("np.tril(np.ones((n, n)))", "np.tril(np.ones((n, n)), -1)"),
    "read_before_update": ("        S += kf[..., i, :, None] * v[..., i, None, :]\n        Z += kf[..., i, :]\n        if causal:",
                           "        if causal:"),
    "dropped_normaliser_grad_q": ("+ c[..., i, None] * Z", "+ 0.0 * Z"),
    "dropped_normaliser_grad_k": ("dkf[..., i, :] = np.einsum(\"...dm,...m->...d\", R, v[..., i, :]) + r",
                                  "dkf[..., i, :] = np.einsum(\"...dm,...m->...d\", R, v[..., i, :])"),
    "prefix_instead_of_suffix": ("for i in range(n - 1, -1, -1):", "for i in range(n):"),
    "wrong_sign_normaliser": ("c = -(G * out).sum(axis=-1) / den", "c = (G * out).sum(axis=-1) / den"),
    "missing_phi_prime": ("dq = dqf * phi_prime(q)", "dq = dqf"),
    "phi_prime_wrong_branch": ("np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))",
                               "np.where(x > 0.0, 1.0, 1.0 + 0.0 * x)"),
    "transposed_state_in_dv": ("dv[..., i, :] = np.einsum(\"...dm,...d->...m\", R, kf[..., i, :])",
                               "dv[..., i, :] = np.einsum(\"...dm,...d->...m\", R[..., ::-1, :], kf[..., i, :])"),
    "decode_update_missing_z": ("    Z = _f64(Z) + kf\n", "    Z = _f64(Z)\n"),
    "prefix_state_drops_feature_map": ("    kf = phi(k)\n    v = _f64(v)\n    S = np.swapaxes",
                                       "    kf = _f64(k)\n    v = _f64(v)\n    S = np.swapaxes"),
    "state_ignored_in_denominator": ("        den = den + (qf * _f64(Z0)[..., None, :]).sum(axis=-1)\n", ""),
    "carried_state_dropped_in_prefix_sweep": ("        S = np.zeros(lead + (d, m)) if S0 is None else _f64(S0).copy()\n",
                                             "        S = np.zeros(lead + (d, m))\n"),
    "state_gradient_misses_normaliser": ("    return dq, dk, dv, R, r, out, den", "    return dq, dk, dv, R, 0.0 * r, out, den"),
    "noncausal_dq_uses_zero_state": ("dqf = np.einsum(\"...dm,...nm->...nd\", S_N, g) + c[..., :, None] * Z_N[..., None, :]",
                                     "dqf = np.einsum(\"...dm,...nm->...nd\", S_N, g)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    assert not pins_pass(load_variant(old, new)), f"pins missed mutant {name}"
