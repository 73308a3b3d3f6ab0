"""Plain fp64 CPU oracle for linear attention with the degree-2 polynomial
feature map.

TEST INFRASTRUCTURE ONLY, like ``linattn_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it; it shares no code with the HIP library.

Source: "[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io),
section 2 (linearised attention), "feature map and computation cost", item
(3): the homogeneous degree-2 polynomial kernel k(x, y) = (x^T y)^2 expands
into sum_i sum_j (x_i x_j)(y_i y_j), so its explicit feature map phi(x) has
the C = D^2 coordinates x_i x_j, one per ordered pair (i, j), and linear
attention with it costs O(N D^2 M).  The attention it plugs into is the
generalised form ``eq:common`` with sim = k, causally masked as in
``eq:mask`` / ``eq:output`` (S_i = sum_{j<=i} phi(K_j) V_j^T,
Z_i = sum_{j<=i} phi(K_j)).

Readings (also listed in the design notes):

* phi(x)[i D + j] = x_i x_j (row-major over the ordered pairs, as the page
  enumerates them); no scaling, no symmetric reduction to D(D+1)/2.
* The denominator sum_j (Q_i^T K_j)^2 is >= 0 and is 0 only when every term
  is 0 -- then the numerator is 0 too.  The pages are silent; no epsilon is
  added (it would bias every row), and a row whose denominator is exactly 0
  reads as 0 (0/0 := 0), with zero gradient through it.
* No 1/sqrt(D) inside the kernel (the workloads pre-scale Q and K).
* Gradients (the pages give none for this kernel) by the chain rule through
  the masked quadratic form; pinned by central finite differences.

Every function works in float64 on arrays whose last two axes are (tokens,
features); leading axes are carried along.

Parity status: every function is pinned in ``tests/test_poly_oracle.py``
(the feature identity, a hand-worked example, the two forms and scalar loops
against each other, zero denominators, sign and scale invariance, state
continuation and decode, finite differences, the Euler identities of the
gradients, and eight planted mistakes); none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = ["phi2", "forward_quadratic", "forward_recurrent", "forward_bruteforce", "prefix_state", "decode_step",
           "backward", "fd_grad"]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def phi2(x):
    """The explicit feature map: [..., D] -> [..., D*D], phi[i D + j] = x_i x_j."""
    x = _f64(x)
    d = x.shape[-1]
    return (x[..., :, None] * x[..., None, :]).reshape(x.shape[:-1] + (d * d,))


def _safe_div(num, den):
    """num / den per row, 0 where den == 0 (then num == 0 as well)."""
    zero = den == 0
    return np.where(zero[..., None], 0.0, num / np.where(zero, 1.0, den)[..., None])


# --------------------------------------------------------------------------
# The definition: eq:common with sim(q, k) = (q^T k)^2, causal per eq:mask.
# --------------------------------------------------------------------------
def forward_quadratic(q, k, v, causal=True):
    """Return (out, den): out_i = sum_j w_ij v_j / den_i, w_ij = (q_i . k_j)^2
    over j <= i (causal) or all j, den_i = sum_j w_ij."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[-2]
    w = (q @ np.swapaxes(k, -1, -2)) ** 2
    if causal:
        w = w * np.tril(np.ones((n, n)))
    den = w.sum(-1)
    return _safe_div(w @ v, den), den


# --------------------------------------------------------------------------
# The linear form with the explicit D^2 features (eq:output): S_i, Z_i.
# --------------------------------------------------------------------------
def forward_recurrent(q, k, v, causal=True, S0=None, Z0=None):
    """Return (out, den, S_N, Z_N) through explicit features, token by token
    (causal) or from the totals (non-causal).  Small D only (C = D^2)."""
    fq, fk, v = phi2(q), phi2(k), _f64(v)
    lead = fq.shape[:-2]
    n, c = fq.shape[-2:]
    m = v.shape[-1]
    S = np.zeros(lead + (c, m)) if S0 is None else _f64(S0).copy()
    Z = np.zeros(lead + (c,)) if Z0 is None else _f64(Z0).copy()
    if not causal:
        S = S + np.einsum("...nc,...nm->...cm", fk, v)
        Z = Z + fk.sum(-2)
        num = np.einsum("...nc,...cm->...nm", fq, S)
        den = np.einsum("...nc,...c->...n", fq, Z)
        return _safe_div(num, den), den, S, Z
    num = np.empty(lead + (n, m))
    den = np.empty(lead + (n,))
    for t in range(n):
        S = S + fk[..., t, :, None] * v[..., t, None, :]
        Z = Z + fk[..., t, :]
        num[..., t, :] = np.einsum("...c,...cm->...m", fq[..., t, :], S)
        den[..., t] = np.einsum("...c,...c->...", fq[..., t, :], Z)
    return _safe_div(num, den), den, S, Z


def forward_bruteforce(q, k, v, causal=True):
    """Scalar loops over one head (q, k: [N, D]; v: [N, M])."""
    n, d = len(q), len(q[0])
    m = len(v[0])
    out = []
    for i in range(n):
        num = [0.0] * m
        den = 0.0
        for j in range(i + 1 if causal else n):
            s = 0.0
            for a in range(d):
                s += float(q[i][a]) * float(k[j][a])
            w = s * s
            den += w
            for c in range(m):
                num[c] += w * float(v[j][c])
        out.append([x / den if den != 0.0 else 0.0 for x in num])
    return np.array(out)


def prefix_state(k, v):
    """(S, Z) after the given tokens: S = sum_j phi(k_j) v_j^T [.., D^2, M],
    Z = sum_j phi(k_j) [.., D^2]."""
    fk = phi2(k)
    return np.einsum("...nc,...nm->...cm", fk, _f64(v)), fk.sum(-2)


def decode_step(S, Z, q, k, v):
    """One recurrent step per head (section 4's loop with phi = phi2): update
    S, Z with the new token, then read.  S [.., D^2, M], Z [.., D^2]; q, k
    [.., D]; v [.., M].  Returns (S, Z, out)."""
    fq, fk = phi2(q), phi2(k)
    S = _f64(S) + fk[..., :, None] * _f64(v)[..., None, :]
    Z = _f64(Z) + fk
    num = np.einsum("...c,...cm->...m", fq, S)
    den = np.einsum("...c,...c->...", fq, Z)
    return S, Z, _safe_div(num[..., None, :], den[..., None])[..., 0, :]


# --------------------------------------------------------------------------
# Backward of L = sum(dout * out) through the masked quadratic form, by the
# chain rule.  With s_ij = q_i . k_j, w_ij = s_ij^2 (masked), den_i, out_i:
#   g_i = dout_i / den_i,  c_i = -(dout_i . out_i) / den_i,
#   dL/dw_ij = g_i . v_j + c_i,   dL/ds_ij = 2 s_ij (g_i . v_j + c_i),
#   dq_i = sum_j dL/ds_ij k_j,  dk_j = sum_i dL/ds_ij q_i,
#   dv_j = sum_i w_ij g_i.
# Rows with den_i = 0 have g_i = c_i = 0 (their output is the constant 0).
# --------------------------------------------------------------------------
def backward(q, k, v, dout, causal=True):
    """Return (dq, dk, dv, out, den)."""
    q, k, v, G = _f64(q), _f64(k), _f64(v), _f64(dout)
    n = q.shape[-2]
    s = q @ np.swapaxes(k, -1, -2)
    mask = np.tril(np.ones((n, n))) if causal else np.ones((n, n))
    w = s * s * mask
    den = w.sum(-1)
    out = _safe_div(w @ v, den)
    zero = den == 0
    inv = np.where(zero, 0.0, 1.0 / np.where(zero, 1.0, den))
    g = G * inv[..., None]
    c = -(G * out).sum(-1) * inv
    dw = g @ np.swapaxes(v, -1, -2) + c[..., None]
    ds = 2.0 * s * dw * mask
    dq = ds @ k
    dk = np.swapaxes(ds, -1, -2) @ q
    dv = np.swapaxes(w, -1, -2) @ g
    return dq, dk, dv, out, den


def fd_grad(q, k, v, dout, causal=True, h: float = 1e-6):
    """Central finite differences of L = sum(dout * out) through
    forward_quadratic; tiny inputs only."""
    arrs = [_f64(q).copy(), _f64(k).copy(), _f64(v).copy()]
    G = _f64(dout)

    def loss():
        return float((G * forward_quadratic(arrs[0], arrs[1], arrs[2], causal)[0]).sum())

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
