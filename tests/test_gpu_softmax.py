"""GPU parity of the softmax-attention baselines against the fp64 oracle,
through the C ABI.

[W] "[Paper walkthrough] Transformers are RNNs", section 1, eq:softmax
(scale 1/sqrt(D)); [T] "Transformer study notes (4)", section
"FlashAttention" (the blockwise update the forward kernel runs); [X] "The
deep link between Transformer and RNN", section 3 (the KV-cache step).
Inputs: q, k, v iid N(0,1)/sqrt(D) unless stated; the oracle sees exactly
the tensors the GPU consumed.  Tolerances: bf16 rel-L2 2e-2 and within 3x of
the bf16 rounding of the exact result; fp32 rel-L2 1e-5; lse absolute 2e-3.
"""

import sys

import numpy as np
import pytest
import torch

import kernelized_causal_attention_amd as la
from oracle import softmax_oracle as so
from workloads import numpy_inputs, rel_l2, to_torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[softmax]", *a, file=sys.stderr, flush=True)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(y, ref, what, factor=3.0):
    e = rel_l2(f64(y), ref)
    e_round = rel_l2(f64(torch.from_numpy(ref).float().to(torch.bfloat16)), ref)
    say(f"{what}: rel-L2 {e:.2e} (bf16 rounding of the exact result {e_round:.2e})")
    assert e < 2e-2
    assert e < max(factor * e_round, 1e-3), (e, e_round)


SHAPES = [(1, 1, 1, 64), (1, 2, 63, 64), (2, 1, 128, 64), (1, 1, 129, 64), (2, 3, 333, 64), (1, 2, 1000, 64),
          (1, 1, 127, 128), (1, 2, 700, 128)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_softmax_forward_matches_oracle(shape, causal):
    B, H, N, D = shape
    q, k, v, _ = numpy_inputs(B, H, N, D, D, seed=N + D + 2, scale=1.0 / np.sqrt(D))
    tq, tk, tv = (to_torch(x, "bf16", DEV) for x in (q, k, v))
    out, lse = la.softmax_forward(tq, tk, tv, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    ref, rlse = so.attention(f64(tq), f64(tk), f64(tv), causal)
    check(out, ref, f"forward {shape} causal={causal}")
    assert np.abs(f64(lse) - rlse).max() < 2e-3


def test_softmax_large_scores():
    # unscaled q, k (scores of size D): the running maximum keeps every
    # exponent <= 0
    B, H, N, D = 1, 2, 300, 64
    q, k, v, _ = numpy_inputs(B, H, N, D, D, seed=5, scale=1.0)
    tq, tk, tv = (to_torch(x, "bf16", DEV) for x in (q * 4.0, k, v))
    out = la.softmax_forward(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    check(out, so.attention(f64(tq), f64(tk), f64(tv))[0], "large scores", factor=4.0)


def test_softmax_forward_workload_sampled_heads():
    B, H, N, D = 8, 16, 8192, 64
    gen = torch.Generator(device=DEV).manual_seed(15)
    mk = lambda: (torch.randn(B, H, N, D, device=DEV, generator=gen) / np.sqrt(D)).to(torch.bfloat16)
    tq, tk, tv = mk(), mk(), mk()
    out = la.softmax_forward(tq, tk, tv)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (7, 15)):
        check(out[b, h], so.attention(f64(tq[b, h]), f64(tk[b, h]), f64(tv[b, h]))[0], f"workload head ({b}, {h})")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("L0", [0, 37, 300])
def test_kv_cache_steps_match_causal_rows(D, dt, L0):
    B, H, steps = 2, 3, 12
    N = L0 + steps
    q, k, v, _ = numpy_inputs(B, H, N, D, D, seed=D + L0, scale=1.0 / np.sqrt(D))
    tq, tk, tv = (to_torch(x, dt, DEV) for x in (q, k, v))
    cap = N + 5
    kc = torch.zeros(B, H, cap, D, dtype=tq.dtype, device=DEV)
    vc = torch.zeros(B, H, cap, D, dtype=tq.dtype, device=DEV)
    kc[:, :, :L0] = tk[:, :, :L0]
    vc[:, :, :L0] = tv[:, :, :L0]
    say(f"kv-cache D={D} {dt} L0={L0}")
    outs = [la.softmax_decode_step(kc, vc, L0 + t, tq[:, :, L0 + t].contiguous(), tk[:, :, L0 + t].contiguous(),
                                   tv[:, :, L0 + t].contiguous()) for t in range(steps)]
    torch.cuda.synchronize()
    ref = so.attention(f64(tq), f64(tk), f64(tv))[0][:, :, L0:]
    y = torch.stack(outs, dim=2)
    if dt == "f32":
        assert rel_l2(f64(y), ref) < 1e-5
    else:
        check(y, ref, f"kv-cache D={D} L0={L0}")
    # the steps appended their tokens
    assert torch.equal(kc[:, :, :N], tk) and torch.equal(vc[:, :, :N], tv)


def test_kv_cache_rejects_full_cache():
    B, H, D = 1, 1, 64
    kc = torch.zeros(B, H, 4, D, device=DEV)
    vc = torch.zeros(B, H, 4, D, device=DEV)
    x = torch.randn(B, H, D, device=DEV)
    with pytest.raises(la.LinAttnError, match="INVALID"):
        la.softmax_decode_step(kc, vc, 4, x, x.clone(), x.clone())
