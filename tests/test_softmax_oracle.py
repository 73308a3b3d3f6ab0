"""Pins for the softmax-attention baseline oracle, against what the pages and
the mathematics fix.

Sources: [W] "[Paper walkthrough] Transformers are RNNs", section 1,
eq:softmax; [T] "Transformer study notes (4)", section "FlashAttention" (the
blockwise m / l / a update and its worked example, stored with its citation
in tests/golden/online_softmax_toy.json); [X] "The deep link between
Transformer and RNN", section 3 (the KV-cache loop).
"""

import json
import math
import os
import types

import numpy as np
import pytest

from oracle import softmax_oracle as so
from workloads import numpy_inputs, rel_l2

GOLD = os.path.join(os.path.dirname(__file__), "golden", "online_softmax_toy.json")


def test_page_worked_example():
    g = json.load(open(GOLD))
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    o, trace = so.online_blocks(g["scores"], g["values"], g["block"])
    p = g["printed"]
    assert abs(o[0] - p["out"]) <= tol
    (m1, l1, a1), (m2, l2, a2) = trace
    assert m1 == p["m1"] and m2 == p["m2"]
    assert abs(l1 - p["l1"]) <= tol and abs(a1[0] - p["a1"]) <= tol
    assert abs(l2 - p["l2"]) <= tol and abs(a2[0] - p["a2"]) <= tol
    # the direct softmax of the same scores gives the same number
    s = np.array(g["scores"])
    w = np.exp(s) / np.exp(s).sum()
    assert abs(w @ np.array(g["values"]) - p["out"]) <= tol


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("block", [1, 3, 4, 16])
def test_blocked_equals_direct(causal, block):
    q, k, v, _ = numpy_inputs(1, 2, 11, 4, 3, seed=31, scale=1.0)
    np.testing.assert_allclose(so.attention_blocked(q, k, v, causal, block), so.attention(q, k, v, causal)[0],
                               rtol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_bruteforce(causal):
    q, k, v, _ = numpy_inputs(1, 1, 9, 5, 2, seed=32, scale=1.0)
    np.testing.assert_allclose(so.attention(q, k, v, causal)[0][0, 0],
                               so.attention_bruteforce(q[0, 0], k[0, 0], v[0, 0], causal), rtol=1e-12)


def test_closed_forms_and_invariance():
    q, k, v, _ = numpy_inputs(1, 2, 10, 4, 3, seed=33, scale=1.0)
    # K = 0: uniform weights -> running mean of V (causal), global mean otherwise
    z = np.zeros_like(k)
    csum = np.cumsum(v, axis=-2) / np.arange(1, 11)[:, None]
    np.testing.assert_allclose(so.attention(q, z, v)[0], csum, rtol=1e-12)
    np.testing.assert_allclose(so.attention(q, z, v, causal=False)[0], np.broadcast_to(v.mean(-2, keepdims=True), v.shape),
                               rtol=1e-12)
    # shifting every key by one vector adds a per-row constant to the scores
    b = np.array([0.7, -1.3, 2.0, 0.1])
    np.testing.assert_allclose(so.attention(q, k + b, v)[0], so.attention(q, k, v)[0], rtol=1e-10)
    # the first row attends only to itself
    np.testing.assert_allclose(so.attention(q, k, v)[0][..., 0, :], v[..., 0, :], rtol=1e-14)
    # lse is the log of the row's normaliser, 1/sqrt(D) scaled
    s = (q @ np.swapaxes(k, -1, -2)) / 2.0
    want = np.log(np.where(np.tril(np.ones((10, 10))) > 0, np.exp(s), 0.0).sum(-1))
    np.testing.assert_allclose(so.attention(q, k, v)[1], want, rtol=1e-12)


def test_large_scores_stay_finite():
    # max subtraction: scores near 1000 do not overflow
    q = np.full((1, 3, 4), 40.0)
    k = np.full((1, 3, 4), 25.0)
    k[0, 1] = 26.0
    v = np.arange(6.0).reshape(1, 3, 2)
    out = so.attention(q, k, v)[0]
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out[0, 2], v[0, 1], rtol=1e-12)  # key 1 wins by 40 * 4 / 2 = 80


def test_kv_cache_steps_equal_causal_rows():
    q, k, v, _ = numpy_inputs(2, 2, 12, 4, 3, seed=34, scale=1.0)
    full = so.attention(q, k, v)[0]
    kc, vc = k[..., :5, :], v[..., :5, :]
    for t in range(5, 12):
        kc, vc, o = so.kv_decode_step(kc, vc, q[..., t, :], k[..., t, :], v[..., t, :])
        np.testing.assert_allclose(o, full[..., t, :], rtol=1e-12)
    assert kc.shape[-2] == 12


# ---------------------------------------------------------- mutants -------
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "softmax_oracle.py")


def load_variant(old, new):
    text = open(SRC).read()
    assert old in text, old
    mod = types.ModuleType("softmax_mutant")
    exec(compile(text.replace(old, new), "softmax_mutant", "exec"), mod.__dict__)
    return mod


def pins_pass(o) -> bool:
    g = json.load(open(GOLD))
    out, trace = o.online_blocks(g["scores"], g["values"], g["block"])
    if abs(out[0] - g["printed"]["out"]) > 5e-5 or abs(trace[0][1] - g["printed"]["l1"]) > 5e-5:
        return False
    q, k, v, _ = numpy_inputs(1, 1, 8, 4, 2, seed=35, scale=1.0)
    direct = o.attention(q, k, v)[0]
    if not np.allclose(direct[0, 0], so.attention_bruteforce(q[0, 0], k[0, 0], v[0, 0]), rtol=1e-10):
        return False
    if not np.allclose(o.attention_blocked(q, k, v, True, 3), direct, rtol=1e-10):
        return False
    qq = np.full((1, 3, 4), 40.0)
    kk = np.full((1, 3, 4), 25.0)
    with np.errstate(all="ignore"):
        if not np.isfinite(o.attention(qq, kk, np.ones((1, 3, 2)))[0]).all():
            return False
    kc, vc = k[..., :3, :], v[..., :3, :]
    for t in range(3, 8):
        kc, vc, od = o.kv_decode_step(kc, vc, q[..., t, :], k[..., t, :], v[..., t, :])
        if not np.allclose(od, direct[..., t, :], rtol=1e-10):
            return False
    return True


SOFTMAX_MUTANTS = {
    "no_scale": ("scale = 1.0 / math.sqrt(d) if scale is None else scale", "scale = 1.0 if scale is None else scale"),
    "strict_mask": ("np.tril(np.ones((n, k.shape[-2]), dtype=bool))", "np.tril(np.ones((n, k.shape[-2]), dtype=bool), -1)"),
    "no_max_subtraction": ("e = np.exp(s - m)", "e = np.exp(s)"),
    "rescale_sign": ("r = math.exp(m - m_new) if m != -np.inf else 0.0", "r = math.exp(m_new - m) if m != -np.inf else 0.0"),
    "a_not_rescaled": ("a = r * a + p @ vb", "a = a + p @ vb"),
    "attend_before_append": ("out = attention(_f64(q)[..., None, :], kc, vc, causal=False)",
                             "out = attention(_f64(q)[..., None, :], _f64(k_cache), _f64(v_cache), causal=False)"),
}


def test_unmodified_softmax_copy_passes():
    assert pins_pass(load_variant("import math", "import math"))


@pytest.mark.parametrize("name", sorted(SOFTMAX_MUTANTS))
def test_softmax_mutant_is_caught(name):
    assert not pins_pass(load_variant(*SOFTMAX_MUTANTS[name])), name
