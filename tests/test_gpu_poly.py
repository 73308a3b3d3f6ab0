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


# ------------------------------------------- linear form: state, decode ----
@pytest.mark.parametrize("shape", [(1, 2, 200, 64), (2, 1, 65, 64), (1, 1, 130, 128)])
def test_poly_prefix_state_matches_oracle(shape):
    # S = sum_t phi(k_t) v_t^T over the D^2 features (one bf16 rounding of
    # each product), Z = sum_t phi(k_t) in fp32
    B, H, N, D = shape
    _, tk, tv, _ = case(B, H, N, D, seed=N + 21)
    S, Z = la.poly_prefix_state(tk, tv)
    torch.cuda.synchronize()
    rS, rZ = po.prefix_state(f64(tk), f64(tv))
    eS, eZ = rel_l2(f64(S), rS), rel_l2(f64(Z), rZ)
    say(f"prefix state {shape}: S rel-L2 {eS:.2e}, Z rel-L2 {eZ:.2e}")
    assert eS < 2e-3
    assert eZ < 1e-5


@pytest.mark.parametrize("D", [64, 128])
def test_poly_prefill_then_decode(D):
    # the prefix state continues the sequence in decode steps; rows equal the
    # masked quadratic form over all the tokens
    B, H, N, a = 2, 2, 220, 200
    tq, tk, tv, _ = case(B, H, N, D, seed=D + 5)
    S, Z = la.poly_prefix_state(tk[:, :, :a].contiguous(), tv[:, :, :a].contiguous())
    outs = [la.poly_decode_step(S, Z, tq[:, :, t].contiguous(), tk[:, :, t].contiguous(), tv[:, :, t].contiguous())
            for t in range(a, N)]
    torch.cuda.synchronize()
    ref = po.forward_quadratic(f64(tq), f64(tk), f64(tv))[0][:, :, a:]
    check(torch.stack(outs, dim=2), ref, f"prefill then decode D={D}")


@pytest.mark.parametrize("dm", [(16, 8), (32, 40), (64, 64), (8, 1)])
def test_poly_decode_steps_fp32_match_oracle(dm):
    # fp32 steps from an fp32 state built by the oracle (vector and scalar
    # kernel paths)
    D, M = dm
    B, H, N = 2, 3, 10
    q, k, v, _ = numpy_inputs(B, H, N, D, M, seed=D * M, scale=1.0 / np.sqrt(D))
    S0, Z0 = po.prefix_state(k[:, :, :4], v[:, :, :4])
    S = torch.tensor(S0, dtype=torch.float32, device=DEV)
    Z = torch.tensor(Z0, dtype=torch.float32, device=DEV)
    tq, tk, tv = (to_torch(x, "f32", DEV) for x in (q, k, v))
    rS, rZ = S0, Z0
    for t in range(4, N):
        o = la.poly_decode_step(S, Z, tq[:, :, t].contiguous(), tk[:, :, t].contiguous(), tv[:, :, t].contiguous())
        rS, rZ, ro = po.decode_step(rS, rZ, f64(tq[:, :, t]), f64(tk[:, :, t]), f64(tv[:, :, t]))
        torch.cuda.synchronize()
        assert rel_l2(f64(o), ro) < 1e-5
    assert rel_l2(f64(S), rS) < 1e-6
    assert rel_l2(f64(Z), rZ) < 1e-6


def test_poly_decode_zero_query_reads_zero():
    B, H, D, M = 1, 2, 16, 8
    S = torch.zeros(B, H, D * D, M, device=DEV)
    Z = torch.zeros(B, H, D * D, device=DEV)
    k = torch.randn(B, H, D, device=DEV)
    v = torch.randn(B, H, M, device=DEV)
    o = la.poly_decode_step(S, Z, torch.zeros(B, H, D, device=DEV), k, v)
    torch.cuda.synchronize()
    assert torch.all(o == 0)


def test_poly_decode_rejects_non_power_of_two():
    B, H, D, M = 1, 1, 48, 8
    S = torch.zeros(B, H, D * D, M, device=DEV)
    Z = torch.zeros(B, H, D * D, device=DEV)
    x = torch.randn(B, H, D, device=DEV)
    with pytest.raises(la.LinAttnError, match="UNSUPPORTED"):
        la.poly_decode_step(S, Z, x, x.clone(), torch.randn(B, H, M, device=DEV))
