"""GPU parity of the degree-2 polynomial-kernel attention against the fp64
oracle, through the C ABI.

"[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io), section 2,
"feature map and computation cost", item (3): sim(q, k) = (q^T k)^2.
Inputs: q, k, v iid N(0,1)/sqrt(D) (bf16), dout iid N(0,1); the oracle sees
exactly the tensors the GPU consumed.  Tolerance: rel-L2 2e-2 (bf16 inputs,
fp32 accumulation) and within 3x (outputs) or 4x (gradients) of the bf16
rounding of the exact result; den (fp32) rel-L2 1e-4.
"""

import sys

import numpy as np
import pytest
import torch

import kernelized_causal_attention_amd as la
from oracle import poly_oracle as po
from workloads import numpy_inputs, rel_l2, to_torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[poly]", *a, file=sys.stderr, flush=True)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def case(B, H, N, D, seed):
    q, k, v, g = numpy_inputs(B, H, N, D, D, seed=seed, scale=1.0 / np.sqrt(D))
    return tuple(to_torch(x, "bf16", DEV) for x in (q, k, v)) + (to_torch(g, "bf16", DEV),)


def check(y, ref, what, factor=3.0, floor=1e-3):
    e = rel_l2(f64(y), ref)
    e_round = rel_l2(f64(torch.from_numpy(ref).float().to(torch.bfloat16)), ref)
    say(f"{what}: rel-L2 {e:.2e} (bf16 rounding of the exact result {e_round:.2e})")
    assert e < 2e-2
    assert e < max(factor * e_round, floor), (e, e_round)


SHAPES = [(1, 1, 1, 64), (1, 2, 63, 64), (2, 1, 128, 64), (1, 1, 129, 64), (2, 3, 333, 64), (1, 2, 1000, 64),
          (1, 1, 127, 128), (1, 2, 700, 128)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_poly_forward_matches_oracle(shape, causal):
    B, H, N, D = shape
    tq, tk, tv, _ = case(B, H, N, D, seed=N + D)
    out, den = la.poly_forward(tq, tk, tv, causal=causal, return_den=True)
    torch.cuda.synchronize()
    ref, rden = po.forward_quadratic(f64(tq), f64(tk), f64(tv), causal)
    check(out, ref, f"forward {shape} causal={causal}")
    assert rel_l2(f64(den), rden) < 1e-4


def test_poly_zero_denominator_rows_read_zero():
    # q rows set to 0: every weight of those rows is 0 -> out 0, den 0
    tq, tk, tv, _ = case(1, 2, 200, 64, seed=9)
    tq[:, :, 0] = 0
    tq[:, :, 150] = 0
    out, den = la.poly_forward(tq, tk, tv, return_den=True)
    torch.cuda.synchronize()
    assert torch.all(out[:, :, 0] == 0) and torch.all(out[:, :, 150] == 0)
    assert torch.all(den[:, :, 0] == 0) and torch.all(den[:, :, 150] == 0)
    assert torch.isfinite(out.float()).all()
    check(out, po.forward_quadratic(f64(tq), f64(tk), f64(tv))[0], "zero rows")


def test_poly_forward_workload_sampled_heads():
    # the fwd+bwd workload's shape (B=8, H=16, N=8192, D=M=64) in the launch
    # configuration the benchmark times; the oracle checks two heads
    B, H, N, D = 8, 16, 8192, 64
    gen = torch.Generator(device=DEV).manual_seed(12)
    mk = lambda: (torch.randn(B, H, N, D, device=DEV, generator=gen) / np.sqrt(D)).to(torch.bfloat16)
    tq, tk, tv = mk(), mk(), mk()
    out, den = la.poly_forward(tq, tk, tv, return_den=True)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (7, 15)):
        ref, rden = po.forward_quadratic(f64(tq[b, h]), f64(tk[b, h]), f64(tv[b, h]))
        check(out[b, h], ref, f"workload head ({b}, {h})")
        assert rel_l2(f64(den[b, h]), rden) < 1e-4


def test_poly_rejects_unsupported():
    tq, tk, tv, _ = case(1, 1, 64, 64, seed=1)
    with pytest.raises(la.LinAttnError, match="UNSUPPORTED"):
        la.poly_forward(tq.float(), tk.float(), tv.float())


# ------------------------------------------------------------ backward ----
def check_grads(got, want, what):
    """dq and dk vanish identically where every row has one key (N = 1: out
    is that key's value whatever q and k are); there the device result must
    be small against dv instead."""
    scale = np.linalg.norm(want[2].ravel())
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        if np.linalg.norm(b.ravel()) <= 1e-9 * scale:
            e = np.linalg.norm(f64(a).ravel()) / scale
            say(f"{what} {name}: exact gradient 0, |got| / |dv| = {e:.2e}")
            assert e < 1e-3
        else:
            # floor: a gradient carries two bf16 roundings (weight and g) even
            # where the exact one is representable (N = 1: dv = dout)
            check(a, b, f"{what} {name}", factor=4.0, floor=5e-3)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_poly_backward_matches_oracle(shape, causal):
    B, H, N, D = shape
    tq, tk, tv, tg = case(B, H, N, D, seed=N + D + 1)
    out, den = la.poly_forward(tq, tk, tv, causal=causal, return_den=True)
    got = la.poly_backward(tq, tk, tv, out, tg, den, causal=causal)
    torch.cuda.synchronize()
    want = po.backward(f64(tq), f64(tk), f64(tv), f64(tg), causal)[:3]
    check_grads(got, want, f"backward {shape} causal={causal}")


def test_poly_backward_zero_rows():
    tq, tk, tv, tg = case(1, 2, 300, 64, seed=13)
    tq[:, :, 5] = 0
    tq[:, :, 200] = 0
    out, den = la.poly_forward(tq, tk, tv, return_den=True)
    dq, dk, dv = la.poly_backward(tq, tk, tv, out, tg, den)
    torch.cuda.synchronize()
    assert torch.all(dq[:, :, 5] == 0) and torch.all(dq[:, :, 200] == 0)
    check_grads((dq, dk, dv), po.backward(f64(tq), f64(tk), f64(tv), f64(tg))[:3], "zero rows")


def test_poly_backward_workload_sampled_heads():
    B, H, N, D = 8, 16, 8192, 64
    gen = torch.Generator(device=DEV).manual_seed(14)
    mk = lambda: (torch.randn(B, H, N, D, device=DEV, generator=gen) / np.sqrt(D)).to(torch.bfloat16)
    tq, tk, tv = mk(), mk(), mk()
    tg = torch.randn(B, H, N, D, device=DEV, generator=gen).to(torch.bfloat16)
    out, den = la.poly_forward(tq, tk, tv, return_den=True)
    got = la.poly_backward(tq, tk, tv, out, tg, den)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (7, 15)):
        want = po.backward(f64(tq[b, h]), f64(tk[b, h]), f64(tv[b, h]), f64(tg[b, h]))[:3]
        check_grads([t[b, h] for t in got], want, f"workload head ({b}, {h})")
