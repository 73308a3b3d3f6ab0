"""GPU parity of decayed / gated linear attention (retention) against the fp64
oracle, through the C ABI.

"08 - Transformer and Variants" (by-xin.github.io), section 1.3.4:
S_t = gamma_t S_{t-1} + k_t v_t^T, y_t = S_t^T q_t.  Inputs: q, k, v iid
N(0,1)/sqrt(D) (bf16), gates gamma_t ~ U(0.6, 1) per token unless stated;
the oracle sees exactly the tensors the GPU consumed.  Tolerance: rel-L2
2e-2 (bf16 inputs, fp32 accumulation) and within 3x of the bf16 rounding of
the exact result.
"""

import sys

import numpy as np
import pytest
import torch

import kernelized_causal_attention_amd as la
from oracle import retention_oracle as ret
from workloads import numpy_inputs, rel_l2, to_torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[retention]", *a, file=sys.stderr, flush=True)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def case(B, H, N, D, seed, lo=0.6, hi=1.0):
    q, k, v, g = numpy_inputs(B, H, N, D, D, seed=seed, scale=1.0 / np.sqrt(D))
    tq, tk, tv, tg = (to_torch(x, "bf16", DEV) for x in (q, k, v, g))
    lg = np.log(np.random.default_rng(seed + 1000).uniform(lo, hi, (B, H, N)))
    tl = torch.tensor(lg, dtype=torch.float32, device=DEV)
    return tq, tk, tv, tg, tl


def check(y, ref, what):
    e = rel_l2(f64(y), ref)
    e_round = rel_l2(f64(torch.from_numpy(ref).float().to(torch.bfloat16)), ref)
    say(f"{what}: rel-L2 {e:.2e} (bf16 rounding of the exact result {e_round:.2e})")
    assert e < 2e-2
    assert e < max(3.0 * e_round, 1e-3), (e, e_round)


RET_SHAPES = [(1, 1, 1, 64), (1, 2, 63, 64), (2, 1, 64, 64), (1, 1, 65, 64), (2, 3, 333, 64), (1, 2, 1000, 64),
              (1, 1, 127, 128), (1, 2, 1100, 128)]


@pytest.mark.parametrize("shape", RET_SHAPES)
@pytest.mark.parametrize("with_state", [False, True])
def test_retention_forward_matches_oracle(shape, with_state):
    B, H, N, D = shape
    tq, tk, tv, _, tl = case(B, H, N, D, seed=N + D + 3)
    S0 = None
    if with_state:
        S0 = np.random.default_rng(N).standard_normal((B, H, D, D)) * 0.3
    tS0 = None if S0 is None else torch.tensor(S0, dtype=torch.float32, device=DEV)
    y, S = la.retention_forward(tq, tk, tv, tl, S0=tS0, return_state=True)
    torch.cuda.synchronize()
    ref, rS = ret.recurrent(f64(tq), f64(tk), f64(tv), f64(tl), S0)
    check(y, ref, f"forward {shape} state={with_state}")
    assert rel_l2(f64(S), rS) < 2e-3


@pytest.mark.parametrize("lo,hi", [(1.0, 1.0), (0.01, 0.2), (0.999, 1.0)])
def test_retention_gate_regimes(lo, hi):
    # no decay (the undecayed sum), strong forgetting, and slow decay over a
    # long head with several segments
    tq, tk, tv, _, tl = case(2, 2, 2000, 64, seed=17, lo=lo, hi=hi)
    y = la.retention_forward(tq, tk, tv, tl)
    torch.cuda.synchronize()
    ref = ret.quadratic(f64(tq), f64(tk), f64(tv), f64(tl))
    check(y, ref, f"gates in [{lo}, {hi}]")


def test_retention_full_reset_gates():
    # gamma_t = 0 (log gamma very negative) at a few tokens: the state
    # restarts there; -1e30 is taken as -80 (gamma ~ 1e-35)
    tq, tk, tv, _, tl = case(1, 2, 300, 64, seed=19)
    tl[:, :, 100] = -1e30
    tl[:, :, 250] = -200.0
    y = la.retention_forward(tq, tk, tv, tl)
    torch.cuda.synchronize()
    lg = np.maximum(f64(tl), -80.0)
    ref = ret.quadratic(f64(tq), f64(tk), f64(tv), lg)
    assert np.isfinite(f64(y)).all()
    check(y, ref, "full resets")


def test_retention_state_continues_and_updates_in_place():
    tq, tk, tv, _, tl = case(2, 2, 900, 64, seed=23)
    a = 371
    S = torch.zeros(2, 2, 64, 64, device=DEV)
    parts = []
    for lo_, hi_ in ((0, a), (a, 900)):
        sl = slice(lo_, hi_)
        parts.append(la.retention_forward(tq[:, :, sl].contiguous(), tk[:, :, sl].contiguous(),
                                          tv[:, :, sl].contiguous(), tl[:, :, sl].contiguous(), S0=S, S_out=S))
    full = la.retention_forward(tq, tk, tv, tl)
    torch.cuda.synchronize()
    ref, rS = ret.recurrent(f64(tq), f64(tk), f64(tv), f64(tl))
    check(torch.cat(parts, dim=2), ref, "two calls with the state carried in place")
    check(full, ref, "one call")
    assert rel_l2(f64(S), rS) < 2e-3


def test_retention_rejects_unsupported():
    tq, tk, tv, _, tl = case(1, 1, 64, 64, seed=1)
    with pytest.raises(la.LinAttnError, match="UNSUPPORTED"):
        la.retention_forward(tq.float(), tk.float(), tv.float(), tl)
