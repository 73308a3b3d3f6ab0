"""Plain, slow, fp64 CPU oracle for causal linear attention with phi = elu + 1.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it; both sides receive the same seeded input
arrays and nothing else.

Every function works in float64 on numpy arrays whose last two axes are
(tokens, features); any leading axes (batch, heads) are carried along.
Nothing here is blocked, fused or reordered beyond what the cited definition
states.

Sources, cited by page title and the section or equation on it:

* [W] "[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io) -- the
  most careful page; its equations carry labels: ``eq:common`` (generalised
  attention), ``eq:linear`` (associativity), ``eq:mask`` (causal masking),
  ``eq:output`` (readout from S_i, Z_i), ``eq:gq``..``eq:gv`` (numerator
  gradients), and section 4 ("Transformers are RNNs", the s_i / z_i
  recurrence).
* [T] "Transformer study notes (4): the basics of linear attention"
  (developer.cloud.tencent.cn) -- section "linear attention".
* [O] "Overview of Linear Attention" (maosong.website) -- section "Linear
  Transformer" and its "Algorithm: Linear transformers with causal masking".
* [X] "The deep link between Transformer and RNN" (xxqk.cn) -- section 3,
  the RNN-mode inference loop (update the state, then read it).

Readings taken where the pages are silent or disagree (each also listed in
the design notes):

* elu's alpha is 1 ([W] section 2 says "usually 1.0"; [T] writes e^x - 1), so
  phi(x) = x + 1 for x > 0 and e^x otherwise.
* The causal mask is inclusive (j <= i) and the state is updated before it
  is read ([W] ``eq:mask``; [O] the forward algorithm; [X] section 3).
* There is no epsilon in the denominator: phi > 0, so the denominator is
  strictly positive for finite inputs ([W] section 2 asks only that sim is
  non-negative).
* Z is a vector of length D ([W] section 3; [T]); one page calls it a scalar,
  which is read as a garble.
* Gradients follow [W]'s summary (prefix sum for phi(Q), suffix sums for
  phi(K) and V).  [O]'s printed gradients swap prefix and suffix and are not
  used.  The denominator and the quotient, which [W] leaves to automatic
  differentiation, are differentiated here by the chain rule (see
  ``backward``).
* Gradients are returned with respect to the raw q, k, v, so phi' is applied.

Parity status: every function below is pinned by tests in
``tests/test_oracle.py`` (two forms of one definition, closed forms, special
cases, invariants and central finite differences); none is "parity
unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "phi",
    "phi_prime",
    "forward_quadratic",
    "forward_recurrent",
    "forward_bruteforce",
    "prefix_state",
    "decode_step",
    "decode_steps",
    "backward",
    "backward_state",
    "fd_grad",
    "fd_grad_state",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Feature map.  [W] section 2 ("feature maps and cost"): phi(x) = elu(x) + 1,
# elu(x) = x for x > 0 and alpha (e^x - 1) for x <= 0, alpha = 1; C = D.
# --------------------------------------------------------------------------
def phi(x) -> np.ndarray:
    """Element-wise phi(x) = elu(x) + 1 with alpha = 1."""
    x = _f64(x)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_prime(x) -> np.ndarray:
    """Derivative of phi: 1 for x > 0, e^x for x <= 0 (continuous at 0)."""
    x = _f64(x)
    return np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))


# --------------------------------------------------------------------------
# Forward, quadratic form: the definition.
# [W] eq:common with sim(q, k) = phi(q)^T phi(k) (section 2), the causal
# mask of eq:mask (section 3), and the denominator phi(Q)(phi(K)^T 1) of
# [X] section 1.  A state (S0, Z0) carried in from earlier tokens ([W]
# section 4 starts from s_0 = z_0 = 0; [X] section 4.2 saves and restores a
# session's state) enters every row as phi(Q_i)^T S0 and phi(Q_i)^T Z0:
# the earlier tokens' terms of the same masked sum.
# --------------------------------------------------------------------------
def forward_quadratic(q, k, v, causal: bool = True, S0=None, Z0=None):
    """Return (out, den) from the O(N^2) masked-sum definition.

    q, k: [..., N, D]; v: [..., N, M].  out: [..., N, M]; den: [..., N].
    S0 [..., D, M], Z0 [..., D] (optional): the state of earlier tokens.
    """
    qf = phi(q)
    kf = phi(k)
    v = _f64(v)
    n = qf.shape[-2]
    w = qf @ np.swapaxes(kf, -1, -2)  # [..., N, N], w_ij = phi(Q_i)^T phi(K_j)
    if causal:
        w = w * np.tril(np.ones((n, n)))  # keep j <= i
    num = w @ v
    den = w.sum(axis=-1)
    if S0 is not None:
        num = num + qf @ _f64(S0)
        den = den + (qf * _f64(Z0)[..., None, :]).sum(axis=-1)
    return num / den[..., None], den


# --------------------------------------------------------------------------
# Forward, recurrent form.  [W] section 3: S_t = S_{t-1} + phi(K_t) V_t^T,
# Z_t = Z_{t-1} + phi(K_t), V'_i = phi(Q_i)^T S_i / phi(Q_i)^T Z_i
# (eq:output); [O] the forward algorithm (update S, then read it).
# Non-causal: [W] eq:linear, the sums run over all N tokens.
# --------------------------------------------------------------------------
def forward_recurrent(q, k, v, causal: bool = True, S0=None, Z0=None):
    """Return (out, den, S_N, Z_N) by walking the tokens one at a time.

    S0, Z0 (optional) are a state carried in from earlier tokens
    ([..., D, M] and [..., D]); the default is s_0 = z_0 = 0 ([W] section 4).
    """
    qf = phi(q)
    kf = phi(k)
    v = _f64(v)
    lead = qf.shape[:-2]
    n, d = qf.shape[-2:]
    m = v.shape[-1]
    S = np.zeros(lead + (d, m)) if S0 is None else _f64(S0).copy()
    Z = np.zeros(lead + (d,)) if Z0 is None else _f64(Z0).copy()
    out = np.empty(lead + (n, m))
    den = np.empty(lead + (n,))
    for i in range(n):
        S += kf[..., i, :, None] * v[..., i, None, :]
        Z += kf[..., i, :]
        if causal:
            num_i = np.einsum("...d,...dm->...m", qf[..., i, :], S)
            den[..., i] = np.einsum("...d,...d->...", qf[..., i, :], Z)
            out[..., i, :] = num_i / den[..., i, None]
    if not causal:
        num = np.einsum("...nd,...dm->...nm", qf, S)
        den = np.einsum("...nd,...d->...n", qf, Z)
        out = num / den[..., None]
    return out, den, S, Z


def forward_bruteforce(q, k, v, causal: bool = True):
    """Scalar loops over [W] eq:common for one head (tiny inputs only).

    q, k: [N, D]; v: [N, M] (nested lists or arrays).  Uses ``math.exp``
    directly rather than ``phi`` above, so it is an independent check of
    both the feature map and the sums.
    """
    q = [[float(x) for x in row] for row in np.asarray(q, dtype=np.float64)]
    k = [[float(x) for x in row] for row in np.asarray(k, dtype=np.float64)]
    v = [[float(x) for x in row] for row in np.asarray(v, dtype=np.float64)]
    n, d, m = len(q), len(q[0]), len(v[0])

    def feat(x):
        return x + 1.0 if x > 0.0 else math.exp(x)

    out = [[0.0] * m for _ in range(n)]
    for i in range(n):
        last = i + 1 if causal else n
        num = [0.0] * m
        den = 0.0
        for j in range(last):
            sim = 0.0
            for t in range(d):
                sim += feat(q[i][t]) * feat(k[j][t])
            den += sim
            for e in range(m):
                num[e] += sim * v[j][e]
        out[i] = [num[e] / den for e in range(m)]
    return np.array(out)


# --------------------------------------------------------------------------
# State from a prefix, and the RNN decode step.
# [W] section 4: s_0 = 0, z_0 = 0, s_i = s_{i-1} + phi(k_i) v_i^T,
# z_i = z_{i-1} + phi(k_i), readout phi(q_i)^T s_i / phi(q_i)^T z_i;
# [X] section 3: the state is updated first, then read.
# --------------------------------------------------------------------------
def prefix_state(k, v):
    """(S, Z) after a prefix: S = sum_j phi(K_j) V_j^T, Z = sum_j phi(K_j)."""
    kf = phi(k)
    v = _f64(v)
    S = np.swapaxes(kf, -1, -2) @ v  # [..., D, M]
    Z = kf.sum(axis=-2)  # [..., D]
    return S, Z


def decode_step(S, Z, q, k, v):
    """One RNN step on a copy of (S, Z); returns (S', Z', out).

    S: [..., D, M]; Z: [..., D]; q, k: [..., D]; v: [..., M].
    """
    qf = phi(q)
    kf = phi(k)
    S = _f64(S) + kf[..., :, None] * _f64(v)[..., None, :]
    Z = _f64(Z) + kf
    num = np.einsum("...d,...dm->...m", qf, S)
    den = np.einsum("...d,...d->...", qf, Z)
    return S, Z, num / den[..., None]


def decode_steps(S, Z, q, k, v):
    """Run ``decode_step`` over a leading step axis: q, k [T, ..., D], v [T, ..., M]."""
    outs = []
    for t in range(np.shape(q)[0]):
        S, Z, o = decode_step(S, Z, q[t], k[t], v[t])
        outs.append(o)
    return S, Z, np.stack(outs)


# --------------------------------------------------------------------------
# Backward.
# Numerator terms: [W] section 3.1, eq:gq (prefix matrix S_i for phi(Q)),
# the phi(K) equation and eq:gv (suffix matrix sum_{j>=i} phi(Q_j) g_j^T).
# Denominator and quotient: left by [W] to autograd; the chain rule gives,
# with num_i = phi(Q_i)^T S_i, den_i = phi(Q_i)^T Z_i, out_i = num_i / den_i
# and G = dL/d out:
#   g_i = dL/d num_i = G_i / den_i,
#   c_i = dL/d den_i = -(G_i . out_i) / den_i,
# so grad phi(Q_i) = S_i g_i + c_i Z_i, and with the suffix sums
#   R_i = sum_{j>=i} phi(Q_j) g_j^T,  r_i = sum_{j>=i} c_j phi(Q_j):
#   grad phi(K_i) = R_i V_i + r_i,  grad V_i = R_i^T phi(K_i).
# The raw-input gradients multiply by phi' (element-wise).
# Non-causal: S_i, Z_i become S_N, Z_N and R_i, r_i become R_1, r_1.
# --------------------------------------------------------------------------
def backward(q, k, v, dout, causal: bool = True):
    """Return (dq, dk, dv, out, den) for the loss L = sum(dout * out)."""
    dq, dk, dv, _, _, out, den = backward_state(q, k, v, dout, None, None, causal)
    return dq, dk, dv, out, den


# With a carried-in state (S0, Z0) the prefix sweep starts from it (S_i and
# Z_i include S0, Z0), and since every row reads S0 and Z0:
#   dL/dS0 = sum_i phi(Q_i) g_i^T = R_1,   dL/dZ0 = sum_i c_i phi(Q_i) = r_1,
# the full suffix sums (non-causal: R, r over all rows, the same sums).
def backward_state(q, k, v, dout, S0, Z0, causal: bool = True):
    """Return (dq, dk, dv, dS0, dZ0, out, den) for L = sum(dout * out) with
    the state (S0, Z0) carried in (None: zero state; dS0, dZ0 still given)."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    G = _f64(dout)
    qf = phi(q)
    kf = phi(k)
    lead = qf.shape[:-2]
    n, d = qf.shape[-2:]
    m = v.shape[-1]

    # Forward sweep: prefix states S_i, Z_i, the outputs and grad phi(Q).
    out, den, S_N, Z_N = forward_recurrent(q, k, v, causal, S0, Z0)
    g = G / den[..., None]
    c = -(G * out).sum(axis=-1) / den
    dqf = np.empty(lead + (n, d))
    if causal:
        S = np.zeros(lead + (d, m)) if S0 is None else _f64(S0).copy()
        Z = np.zeros(lead + (d,)) if Z0 is None else _f64(Z0).copy()
        for i in range(n):
            S += kf[..., i, :, None] * v[..., i, None, :]
            Z += kf[..., i, :]
            dqf[..., i, :] = (
                np.einsum("...dm,...m->...d", S, g[..., i, :]) + c[..., i, None] * Z
            )
    else:
        dqf = np.einsum("...dm,...nm->...nd", S_N, g) + c[..., :, None] * Z_N[..., None, :]

    # Reverse sweep: suffix sums R_i, r_i, then grad phi(K) and grad V.
    dkf = np.empty(lead + (n, d))
    dv = np.empty(lead + (n, m))
    if causal:
        R = np.zeros(lead + (d, m))
        r = np.zeros(lead + (d,))
        for i in range(n - 1, -1, -1):
            R += qf[..., i, :, None] * g[..., i, None, :]
            r += c[..., i, None] * qf[..., i, :]
            dkf[..., i, :] = np.einsum("...dm,...m->...d", R, v[..., i, :]) + r
            dv[..., i, :] = np.einsum("...dm,...d->...m", R, kf[..., i, :])
    else:
        R = np.einsum("...nd,...nm->...dm", qf, g)
        r = np.einsum("...n,...nd->...d", c, qf)
        dkf = np.einsum("...dm,...nm->...nd", R, v) + r[..., None, :]
        dv = np.einsum("...dm,...nd->...nm", R, kf)

    dq = dqf * phi_prime(q)
    dk = dkf * phi_prime(k)
    # R and r now hold the sums over all rows
    return dq, dk, dv, R, r, out, den


def fd_grad(q, k, v, dout, causal: bool = True, h: float = 1e-6):
    """Central finite differences of L = sum(dout * out) through the
    quadratic definition; returns (dq, dk, dv).  For tiny inputs only."""
    arrs = [_f64(q).copy(), _f64(k).copy(), _f64(v).copy()]
    G = _f64(dout)

    def loss():
        o, _ = forward_quadratic(arrs[0], arrs[1], arrs[2], causal)
        return float((G * o).sum())

    grads = []
    for a in arrs:
        gr = np.zeros_like(a)
        flat = a.reshape(-1)
        gflat = gr.reshape(-1)
        for idx in range(flat.size):
            x0 = flat[idx]
            flat[idx] = x0 + h
            lp = loss()
            flat[idx] = x0 - h
            lm = loss()
            flat[idx] = x0
            gflat[idx] = (lp - lm) / (2.0 * h)
        grads.append(gr)
    return tuple(grads)


def fd_grad_state(q, k, v, dout, S0, Z0, causal: bool = True, h: float = 1e-6):
    """Central finite differences of L = sum(dout * out) through the
    quadratic definition with a carried-in state; returns
    (dq, dk, dv, dS0, dZ0).  For tiny inputs only."""
    arrs = [_f64(q).copy(), _f64(k).copy(), _f64(v).copy(), _f64(S0).copy(), _f64(Z0).copy()]
    G = _f64(dout)

    def loss():
        o, _ = forward_quadratic(arrs[0], arrs[1], arrs[2], causal, arrs[3], arrs[4])
        return float((G * o).sum())

    grads = []
    for a in arrs:
        gr = np.zeros_like(a)
        flat = a.reshape(-1)
        gflat = gr.reshape(-1)
        for idx in range(flat.size):
            x0 = flat[idx]
            flat[idx] = x0 + h
            lp = loss()
            flat[idx] = x0 - h
            lm = loss()
            flat[idx] = x0
            gflat[idx] = (lp - lm) / (2.0 * h)
        grads.append(gr)
    return tuple(grads)
