"""Plain fp64 CPU oracle for the softmax-attention baselines (the comparison
method the pages measure linear attention against).

TEST INFRASTRUCTURE ONLY, like ``linattn_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it; it shares no code with the HIP library.

Sources:

* [W] "[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io),
  section 1, ``eq:softmax``: softmax(Q K^T / sqrt(D)) V; ``eq:common`` with
  sim(q, k) = exp(q^T k / sqrt(D)) is the same thing, causally masked as in
  ``eq:mask``.
* [T] "Transformer study notes (4): the basics of linear attention"
  (developer.cloud.tencent.cn), section "FlashAttention": the max-subtracted
  softmax, and the blockwise update of the running maximum m, the rescaled
  denominator l and the unnormalised weighted sum a, with a worked example.
* [X] "The deep link between Transformer and RNN" (xxqk.cn), section 3: the
  KV-cache inference loop (append the new key and value, then attend with
  the new query over every cached position).

Readings (also listed in the design notes):

* The scale is 1/sqrt(D) ([W] ``eq:softmax``; one page divides by d, one
  page omits it in the KV-cache loop -- both read as garbles of 1/sqrt(D)).
* The causal mask is inclusive (j <= i); in the KV-cache loop the new token
  is appended before attending, so it attends to itself.

Every function works in float64 on arrays whose last two axes are (tokens,
features); leading axes are carried along.

Parity status: every function is pinned in ``tests/test_softmax_oracle.py``
(the page's worked example, the two forms against each other, scalar loops,
closed forms and invariances, planted mistakes); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["attention", "attention_bruteforce", "online_blocks", "attention_blocked", "kv_decode_step"]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# The definition ([W] eq:softmax, causal per eq:mask), max-subtracted as [T]
# writes it.  Returns (out, lse) with lse_i = log sum_j exp(s_ij).
# --------------------------------------------------------------------------
def attention(q, k, v, causal=True, scale=None):
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape[-2:]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = (q @ np.swapaxes(k, -1, -2)) * scale
    if causal:
        s = np.where(np.tril(np.ones((n, k.shape[-2]), dtype=bool)), s, -np.inf)
    m = s.max(-1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(-1, keepdims=True)
    return (e / den) @ v, (m + np.log(den))[..., 0]


def attention_bruteforce(q, k, v, causal=True):
    """Scalar loops over one head (q, k: [N, D]; v: [N, M]), own math.exp."""
    n, d = len(q), len(q[0])
    m = len(v[0])
    out = []
    for i in range(n):
        keys = range(i + 1) if causal else range(len(k))
        s = [sum(float(q[i][a]) * float(k[j][a]) for a in range(d)) / math.sqrt(d) for j in keys]
        top = max(s)
        w = [math.exp(x - top) for x in s]
        tot = sum(w)
        out.append([sum(w[t] * float(v[j][c]) for t, j in enumerate(keys)) / tot for c in range(m)])
    return np.array(out)


# --------------------------------------------------------------------------
# [T]'s blockwise update for one query: for each block b of scores s^(b) and
# values V^(b),
#   m_new = max(m_old, max_j s_j),
#   l_new = exp(m_old - m_new) l_old + sum_j exp(s_j - m_new),
#   a_new = exp(m_old - m_new) a_old + sum_j exp(s_j - m_new) v_j,
# and o = a / l at the end.  Returns o and the (m, l, a) after every block.
# --------------------------------------------------------------------------
def online_blocks(scores, values, block):
    s = _f64(scores)
    v = _f64(values)
    if v.ndim == 1:
        v = v[:, None]
    m, l, a = -np.inf, 0.0, np.zeros(v.shape[1])
    trace = []
    for b0 in range(0, len(s), block):
        sb, vb = s[b0:b0 + block], v[b0:b0 + block]
        m_new = max(m, float(sb.max()))
        r = math.exp(m - m_new) if m != -np.inf else 0.0
        p = np.exp(sb - m_new)
        l = r * l + float(p.sum())
        a = r * a + p @ vb
        m = m_new
        trace.append((m, l, a.copy()))
    return a / l, trace


def attention_blocked(q, k, v, causal=True, block=4):
    """The attention rows computed with online_blocks over key blocks."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    d = q.shape[-1]
    lead = q.shape[:-2]
    n = q.shape[-2]
    out = np.empty(lead + (n, v.shape[-1]))
    for idx in np.ndindex(*lead):
        for i in range(n):
            nk = i + 1 if causal else k.shape[-2]
            s = (k[idx][:nk] @ q[idx][i]) / math.sqrt(d)
            out[idx + (i,)] = online_blocks(s, v[idx][:nk], block)[0]
    return out


# --------------------------------------------------------------------------
# [X] section 3's KV-cache step: append (k, v), then attend with q over every
# cached position.  k_cache [.., L, D], v_cache [.., L, M]; q, k [.., D];
# v [.., M].  Returns (k_cache', v_cache', out).
# --------------------------------------------------------------------------
def kv_decode_step(k_cache, v_cache, q, k, v):
    kc = np.concatenate([_f64(k_cache), _f64(k)[..., None, :]], axis=-2)
    vc = np.concatenate([_f64(v_cache), _f64(v)[..., None, :]], axis=-2)
    out = attention(_f64(q)[..., None, :], kc, vc, causal=False)[0][..., 0, :]
    return kc, vc, out
