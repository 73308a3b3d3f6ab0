"""Plain fp64 CPU oracle for decayed / gated linear attention (retention).

TEST INFRASTRUCTURE ONLY, like ``linattn_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it; it shares no code with the HIP library.

Source: "08 - Transformer and Variants" (by-xin.github.io), section 1.3.4
("forgettable linear attention"): RetNet keeps H_t = gamma H_{t-1} + v_t k_t^T
with y_t = H_t q_t and a decay gamma in [0, 1]; gated retention makes the
decay time-varying, gamma_t = sigmoid(W_gamma x_t).  Section 1.3.1 gives the
unrolled sum of the same recurrence without decay.  The page's forms have no
feature map and no normaliser, and are implemented as printed.

Readings (also listed in the design notes):

* The decay is an input per (batch, head, token), passed as log gamma_t <= 0
  (fp64 here, fp32 on the device); RetNet's constant gamma is the case
  log gamma_t = log gamma for every t, and gamma_t = 1 recovers the
  undecayed recurrence of section 1.3.1.  (The page produces gamma_t from
  the token through a learned projection; the projection is outside this
  path, as are W_q, W_k, W_v.)
* The state is stored as S = H^T: S_t = gamma_t S_{t-1} + k_t v_t^T
  ([..., D, M], the same orientation as the linear-attention state), so
  y_t = S_t^T q_t.  A carried-in state S0 is decayed by gamma_1 at the
  first token, as the recurrence says.
* The page gives no gradients; ``backward`` differentiates the recurrence by
  the chain rule (see there) and is pinned by central finite differences.

Every function works in float64 on arrays whose last two axes are
(tokens, features); leading axes are carried along.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["recurrent", "quadratic", "bruteforce", "backward", "fd_grad", "decode_step"]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# The recurrence as printed (section 1.3.4): S_t = gamma_t S_{t-1} + k_t v_t^T,
# y_t = S_t^T q_t.
# --------------------------------------------------------------------------
def recurrent(q, k, v, log_gamma, S0=None):
    """Return (y, S_N) by walking the tokens one at a time.

    q, k: [..., N, D]; v: [..., N, M]; log_gamma: [..., N] (<= 0);
    S0: [..., D, M] or None (zero state)."""
    q, k, v, lg = _f64(q), _f64(k), _f64(v), _f64(log_gamma)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    m = v.shape[-1]
    S = np.zeros(lead + (d, m)) if S0 is None else _f64(S0).copy()
    y = np.empty(lead + (n, m))
    for t in range(n):
        S = np.exp(lg[..., t])[..., None, None] * S + k[..., t, :, None] * v[..., t, None, :]
        y[..., t, :] = np.einsum("...d,...dm->...m", q[..., t, :], S)
    return y, S


# --------------------------------------------------------------------------
# The unrolled sum (the parallel form): with L_i = sum_{l <= i} log gamma_l,
#   y_i = sum_{j <= i} exp(L_i - L_j) (q_i . k_j) v_j + exp(L_i) S0^T q_i,
# section 1.3.1's expansion of H_t with the decays of section 1.3.4 carried
# through each term.
# --------------------------------------------------------------------------
def quadratic(q, k, v, log_gamma, S0=None):
    """Return y from the O(N^2) decayed masked sum."""
    q, k, v, lg = _f64(q), _f64(k), _f64(v), _f64(log_gamma)
    n = q.shape[-2]
    L = np.cumsum(lg, axis=-1)
    # only the terms j <= i exist: exp(L_i - L_j) there (an exponent <= 0);
    # the masked entries are not formed (they would overflow for long gated
    # sequences and turn 0 * inf into NaN)
    keep = np.tril(np.ones((n, n), dtype=bool))
    decay = np.where(keep, np.exp(np.where(keep, L[..., :, None] - L[..., None, :], 0.0)), 0.0)
    w = (q @ np.swapaxes(k, -1, -2)) * decay
    y = w @ v
    if S0 is not None:
        y = y + np.exp(L)[..., None] * (q @ _f64(S0))
    return y


def bruteforce(q, k, v, log_gamma):
    """Scalar loops over one head (q, k: [N, D]; v: [N, M]); own math.exp."""
    n, d = len(q), len(q[0])
    m = len(v[0])
    y = []
    for i in range(n):
        row = [0.0] * m
        for j in range(i + 1):
            dec = 1.0
            for l in range(j + 1, i + 1):
                dec *= math.exp(float(log_gamma[l]))
            s = sum(float(q[i][a]) * float(k[j][a]) for a in range(d)) * dec
            for c in range(m):
                row[c] += s * float(v[j][c])
        y.append(row)
    return np.array(y)


def decode_step(S, q, k, v, log_gamma):
    """One recurrent step per head: S <- gamma S + k v^T, then y = S^T q.
    S [..., D, M]; q, k [..., D]; v [..., M]; log_gamma [...]."""
    S = np.exp(_f64(log_gamma))[..., None, None] * _f64(S) + _f64(k)[..., :, None] * _f64(v)[..., None, :]
    return S, np.einsum("...d,...dm->...m", _f64(q), S)


# --------------------------------------------------------------------------
# Backward of L = sum(dy * y), by the chain rule through the recurrence:
#   dq_i = S_i dy_i                      (S_i: the state after token i)
#   R_i  = sum_{t >= i} exp(L_t - L_i) q_t dy_t^T
#        = q_i dy_i^T + gamma_{i+1} R_{i+1}   (suffix state, reverse sweep)
#   dk_i = R_i v_i,   dv_i = R_i^T k_i,   dS0 = gamma_1 R_1
# and for the decays, since L_m enters row m's terms with + and column m's
# with -,  dL/dL_m = q_m . dq_m - k_m . dk_m, and L_m = sum_{l <= m} log
# gamma_l gives  d log gamma_t = sum_{m >= t} (q_m . dq_m - k_m . dk_m).
# --------------------------------------------------------------------------
def backward(q, k, v, log_gamma, dy, S0=None):
    """Return (dq, dk, dv, dlog_gamma, dS0) for L = sum(dy * y)."""
    q, k, v, lg, G = _f64(q), _f64(k), _f64(v), _f64(log_gamma), _f64(dy)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    m = v.shape[-1]
    S = np.zeros(lead + (d, m)) if S0 is None else _f64(S0).copy()
    dq = np.empty(q.shape)
    for t in range(n):
        S = np.exp(lg[..., t])[..., None, None] * S + k[..., t, :, None] * v[..., t, None, :]
        dq[..., t, :] = np.einsum("...dm,...m->...d", S, G[..., t, :])
    dk = np.empty(k.shape)
    dv = np.empty(v.shape)
    R = np.zeros(lead + (d, m))
    for t in range(n - 1, -1, -1):
        if t < n - 1:
            R = np.exp(lg[..., t + 1])[..., None, None] * R
        R = R + q[..., t, :, None] * G[..., t, None, :]
        dk[..., t, :] = np.einsum("...dm,...m->...d", R, v[..., t, :])
        dv[..., t, :] = np.einsum("...dm,...d->...m", R, k[..., t, :])
    dS0 = np.exp(lg[..., 0])[..., None, None] * R
    per_token = (q * dq).sum(-1) - (k * dk).sum(-1)
    dlg = np.flip(np.cumsum(np.flip(per_token, -1), -1), -1)
    return dq, dk, dv, dlg, dS0


def fd_grad(q, k, v, log_gamma, dy, S0=None, h: float = 1e-6):
    """Central finite differences of L = sum(dy * y) through the quadratic
    form; returns (dq, dk, dv, dlog_gamma[, dS0]).  Tiny inputs only."""
    arrs = [_f64(q).copy(), _f64(k).copy(), _f64(v).copy(), _f64(log_gamma).copy()]
    if S0 is not None:
        arrs.append(_f64(S0).copy())
    G = _f64(dy)

    def loss():
        y = quadratic(arrs[0], arrs[1], arrs[2], arrs[3], arrs[4] if S0 is not None else None)
        return float((G * y).sum())

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
