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
              (1, 1, 127, 128), (1, 2, 1100, 128),
              # nine segments: the decayed scans read a full batch of eight
              # records and a partial one
              (1, 1, 2600, 64)]


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


@pytest.mark.parametrize("N", [300, 3000])
def test_retention_forward_without_state_output(N):
    # S0 given, no S_out: the segment pass skips the last segment, and with a
    # single segment it is not launched (the scan writes S0 into the record);
    # the output must equal the call that also returns the state, bit for bit
    B, H, D = 1, 2, 64
    tq, tk, tv, _, tl = case(B, H, N, D, seed=N + 7)
    assert (la.resolve_plan("retention_forward", B, H, N, D, D, True, "bf16")["segments"] == 1) == (N == 300)
    S0 = torch.tensor(np.random.default_rng(N).standard_normal((B, H, D, D)) * 0.3, dtype=torch.float32,
                      device=DEV)
    want, _ = la.retention_forward(tq, tk, tv, tl, S0=S0, return_state=True)
    got = la.retention_forward(tq, tk, tv, tl, S0=S0)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    ref, _ = ret.recurrent(f64(tq), f64(tk), f64(tv), f64(tl), f64(S0))
    check(got, ref, f"forward without S_out N={N}")


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


# ------------------------------------------------------------ backward ----
# Gradients of L = sum(dy * y) against the oracle's chain rule through the
# recurrence (pinned there by finite differences).  dq, dk, dv are bf16 and
# take the forward's bound; dlog_gamma and dS0 are fp32 outputs built from bf16
# operands and take the bf16 tolerance 2e-2.
def bwd_case(B, H, N, D, seed, lo=0.6, hi=1.0, with_state=False):
    tq, tk, tv, tg, tl = case(B, H, N, D, seed, lo, hi)
    S0 = np.random.default_rng(seed + 7).standard_normal((B, H, D, D)) * 0.3 if with_state else None
    tS0 = None if S0 is None else torch.tensor(S0, dtype=torch.float32, device=DEV)
    return tq, tk, tv, tg, tl, S0, tS0


def check_grads(got, want, what, q=None):
    """dlog_gamma is a reverse sum of q.dq - k.dk; where the exact sum is 0
    (one token and no carried state: the only decay multiplies a zero state)
    its error is taken relative to the size of the q.dq terms instead."""
    names = ("dq", "dk", "dv", "dlog_gamma", "dS0")
    for name, a, b in zip(names, got, want):
        if name in ("dq", "dk", "dv"):
            check(a, b, f"{what} {name}")
        else:
            e_abs = np.linalg.norm((f64(a) - b).ravel())
            nb = np.linalg.norm(b.ravel())
            s = np.linalg.norm((f64(q) * want[0]).sum(-1).ravel()) if (name == "dlog_gamma" and q is not None) else 0
            e = e_abs / nb if nb > 1e-9 * s else e_abs / s
            say(f"{what} {name}: rel-L2 {e:.2e}")
            assert np.isfinite(f64(a)).all()
            assert e < 2e-2, (name, e)


@pytest.mark.parametrize("shape", RET_SHAPES)
@pytest.mark.parametrize("with_state", [False, True])
def test_retention_backward_matches_oracle(shape, with_state):
    B, H, N, D = shape
    tq, tk, tv, tg, tl, S0, tS0 = bwd_case(B, H, N, D, seed=N + D + 5, with_state=with_state)
    say(f"backward {shape} state={with_state}")
    got = la.retention_backward(tq, tk, tv, tl, tg, S0=tS0)
    torch.cuda.synchronize()
    want = ret.backward(f64(tq), f64(tk), f64(tv), f64(tl), f64(tg), S0)
    check_grads(got, want, f"backward {shape} state={with_state}", q=tq)


@pytest.mark.parametrize("lo,hi", [(1.0, 1.0), (0.01, 0.2), (0.999, 1.0)])
def test_retention_backward_gate_regimes(lo, hi):
    tq, tk, tv, tg, tl, _, _ = bwd_case(2, 2, 2000, 64, seed=29, lo=lo, hi=hi)
    say(f"backward gates in [{lo}, {hi}]")
    got = la.retention_backward(tq, tk, tv, tl, tg)
    torch.cuda.synchronize()
    want = ret.backward(f64(tq), f64(tk), f64(tv), f64(tl), f64(tg))
    check_grads(got, want, f"backward gates in [{lo}, {hi}]", q=tq)


def test_retention_backward_full_reset_gates():
    # below -80 a gate is taken as -80 in both passes; the gradient returned
    # there is the one at -80 (where gamma ~ 0 makes it ~ 0 anyway)
    tq, tk, tv, tg, tl, _, _ = bwd_case(1, 2, 300, 64, seed=31)
    tl[:, :, 100] = -1e30
    tl[:, :, 250] = -200.0
    got = la.retention_backward(tq, tk, tv, tl, tg)
    torch.cuda.synchronize()
    lg = np.maximum(f64(tl), -80.0)
    want = ret.backward(f64(tq), f64(tk), f64(tv), lg, f64(tg))
    check_grads(got, want, "backward with full resets", q=tq)


def test_retention_backward_split_sequence_chains_state_gradients():
    # gradients of a sequence cut in two, with the state carried: the second
    # half's dS0 is the gradient the first half receives through S_out; the
    # first half's own dy plus that carried gradient reproduce the gradients
    # of the whole sequence.  Checks dS0 as a seam, against the oracle.
    B, H, N, D, a = 1, 2, 700, 64, 301
    tq, tk, tv, tg, tl, _, _ = bwd_case(B, H, N, D, seed=37)
    sl1, sl2 = slice(0, a), slice(a, N)
    part = lambda t, s: t[:, :, s].contiguous()
    S = torch.zeros(B, H, D, D, device=DEV)
    la.retention_forward(part(tq, sl1), part(tk, sl1), part(tv, sl1), part(tl, sl1), S0=S, S_out=S)
    g2 = la.retention_backward(part(tq, sl2), part(tk, sl2), part(tv, sl2), part(tl, sl2), part(tg, sl2), S0=S)
    torch.cuda.synchronize()
    want = ret.backward(f64(tq), f64(tk), f64(tv), f64(tl), f64(tg))
    for name, got_t, full_t in zip(("dq", "dk", "dv"), g2[:3], want[:3]):
        check(got_t, full_t[:, :, a:], f"second half {name}")
    # the oracle's second half from the oracle's state gives the same dS0
    _, S_a = ret.recurrent(f64(tq)[:, :, :a], f64(tk)[:, :, :a], f64(tv)[:, :, :a], f64(tl)[:, :, :a])
    w2 = ret.backward(f64(tq)[:, :, a:], f64(tk)[:, :, a:], f64(tv)[:, :, a:], f64(tl)[:, :, a:], f64(tg)[:, :, a:],
                      S_a)
    assert rel_l2(f64(g2[4]), w2[4]) < 2e-2
    assert rel_l2(f64(g2[3]), w2[3]) < 2e-2


def test_retention_backward_rejects_unsupported():
    tq, tk, tv, tg, tl, _, _ = bwd_case(1, 1, 64, 64, seed=2)
    with pytest.raises(la.LinAttnError, match="UNSUPPORTED"):
        la.retention_backward(tq.float(), tk.float(), tv.float(), tl, tg.float())


@pytest.mark.parametrize("lo,hi", [(0.01, 0.2), (0.95, 1.0)])
def test_retention_backward_many_heads(lo, hi):
    # 512 heads: the plan gives one 4096-token segment per head, whose gate
    # gradients are anchored at its three inner anchors (every 1024 tokens)
    # and at its end; heads are independent, so the oracle checks four of
    # them (both ends of the batch)
    B, H, N, D = 4, 128, 4096, 64
    plan = la.resolve_plan("retention_backward", B, H, N, D, D, True, "bf16")
    assert plan["segments"] == 1
    gen = torch.Generator(device=DEV).manual_seed(41)
    mk = lambda: (torch.randn(B, H, N, D, device=DEV, generator=gen) / np.sqrt(D)).to(torch.bfloat16)
    tq, tk, tv, tg = mk(), mk(), mk(), mk()
    tl = torch.log(torch.rand(B, H, N, device=DEV, generator=gen) * (hi - lo) + lo).float()
    say(f"backward B={B} H={H} N={N} gates in [{lo}, {hi}]")
    got = la.retention_backward(tq, tk, tv, tl, tg)
    torch.cuda.synchronize()
    for b, hs in ((0, slice(0, 2)), (3, slice(126, 128))):
        want = ret.backward(f64(tq[b, hs]), f64(tk[b, hs]), f64(tv[b, hs]), f64(tl[b, hs]), f64(tg[b, hs]))
        check_grads([t[b, hs] for t in got], want, f"many heads, batch {b} heads {hs.start}..{hs.stop - 1}",
                    q=tq[b, hs])


@pytest.mark.parametrize("D,with_state", [(64, False), (64, True), (128, True)])
def test_retention_backward_inner_anchors_ragged(D, with_state):
    # 256 heads of 2500 tokens: two segments per head (0..1279, 1280..2499),
    # each with one inner anchor (1024 and 2304), the second segment ragged;
    # the oracle checks two heads at each end of the batch, with the
    # forward's saved states and without
    B, H, N = 2, 128, 2500
    plan = la.resolve_plan("retention_backward", B, H, N, D, D, True, "bf16")
    assert plan["segments"] == 2  # of ceil(40 / 2) = 20 chunks = 1280 tokens
    gen = torch.Generator(device=DEV).manual_seed(43)
    mk = lambda: (torch.randn(B, H, N, D, device=DEV, generator=gen) / np.sqrt(D)).to(torch.bfloat16)
    tq, tk, tv, tg = mk(), mk(), mk(), mk()
    tl = torch.log(torch.rand(B, H, N, device=DEV, generator=gen) * 0.4 + 0.6).float()
    tS0 = (torch.randn(B, H, D, D, device=DEV, generator=gen) * 0.3) if with_state else None
    say(f"backward B={B} H={H} N={N} D={D} inner anchors, state={with_state}")
    saved = torch.empty(la.retention_saved_bytes(B, H, N, D, D), dtype=torch.uint8, device=DEV)
    la.retention_forward(tq, tk, tv, tl, S0=tS0, saved=saved)
    with_saved = la.retention_backward(tq, tk, tv, tl, tg, S0=tS0, saved=saved)
    got = la.retention_backward(tq, tk, tv, tl, tg, S0=tS0)
    torch.cuda.synchronize()
    for a, b in zip(with_saved, got):
        assert torch.equal(a, b)
    for b, hs in ((0, slice(0, 2)), (1, slice(126, 128))):
        S0 = None if tS0 is None else f64(tS0[b, hs])
        want = ret.backward(f64(tq[b, hs]), f64(tk[b, hs]), f64(tv[b, hs]), f64(tl[b, hs]), f64(tg[b, hs]), S0)
        check_grads([t[b, hs] for t in got], want, f"inner anchors, batch {b} heads {hs.start}..{hs.stop - 1}",
                    q=tq[b, hs])


# -------------------------------------------------------------- decode ----
DEC_SHAPES = [(2, 3, 64, 64), (1, 2, 128, 128), (2, 1, 48, 40), (1, 1, 256, 64), (1, 2, 7, 1)]


@pytest.mark.parametrize("shape", DEC_SHAPES)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_retention_decode_steps_match_recurrence(shape, dt):
    # token-by-token steps from a random state reproduce the recurrence
    B, H, D, M = shape
    N = 12
    q, k, v, _ = numpy_inputs(B, H, N, D, M, seed=D + M, scale=1.0 / np.sqrt(D))
    tq, tk, tv = (to_torch(x, dt, DEV) for x in (q, k, v))
    lg = np.log(np.random.default_rng(D).uniform(0.5, 1.0, (B, H, N)))
    tl = torch.tensor(lg, dtype=torch.float32, device=DEV)
    S0 = np.random.default_rng(M).standard_normal((B, H, D, M)) * 0.2
    S = torch.tensor(S0, dtype=torch.float32, device=DEV)
    say(f"decode {shape} {dt}")
    ys = [la.retention_decode_step(S, tq[:, :, t].contiguous(), tk[:, :, t].contiguous(), tv[:, :, t].contiguous(),
                                   tl[:, :, t].contiguous()) for t in range(N)]
    torch.cuda.synchronize()
    ref, rS = ret.recurrent(f64(tq), f64(tk), f64(tv), f64(tl), S0)
    y = torch.stack(ys, dim=2)
    if dt == "f32":
        assert rel_l2(f64(y), ref) < 1e-4
    else:
        check(y, ref, f"decode {shape} bf16")
    assert rel_l2(f64(S), rS) < 1e-5


def test_retention_prefill_then_decode():
    # the forward's final state continues the sequence in decode steps
    B, H, N, D, a = 2, 2, 300, 64, 257
    tq, tk, tv, _, tl = case(B, H, N, D, seed=43)
    S = torch.empty(B, H, D, D, device=DEV)
    y1 = la.retention_forward(tq[:, :, :a].contiguous(), tk[:, :, :a].contiguous(), tv[:, :, :a].contiguous(),
                              tl[:, :, :a].contiguous(), S_out=S)
    ys = [la.retention_decode_step(S, tq[:, :, t].contiguous(), tk[:, :, t].contiguous(), tv[:, :, t].contiguous(),
                                   tl[:, :, t].contiguous()) for t in range(a, N)]
    torch.cuda.synchronize()
    ref, rS = ret.recurrent(f64(tq), f64(tk), f64(tv), f64(tl))
    check(torch.cat([y1, torch.stack(ys, dim=2)], dim=2), ref, "prefill then decode")
    assert rel_l2(f64(S), rS) < 2e-3


def test_retention_decode_full_reset():
    # log gamma = -1e30 (taken as -80): the old state is forgotten
    B, H, D, M = 1, 2, 64, 64
    q, k, v, _ = numpy_inputs(B, H, 1, D, M, seed=3, scale=1.0)
    tq, tk, tv = (to_torch(x[:, :, 0], "f32", DEV) for x in (q, k, v))
    S = torch.randn(B, H, D, M, device=DEV)
    y = la.retention_decode_step(S, tq, tk, tv, torch.full((B, H), -1e30, device=DEV))
    torch.cuda.synchronize()
    want_S = f64(tk)[..., :, None] * f64(tv)[..., None, :]
    np.testing.assert_allclose(f64(S), want_S, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(f64(y), np.einsum("bhd,bhdm->bhm", f64(tq), want_S), rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("shape,with_state", [((2, 3, 333, 64), True), ((1, 2, 3000, 64), False),
                                              ((1, 2, 1100, 128), True), ((1, 1, 1, 64), False)])
def test_retention_backward_reads_saved_states(shape, with_state):
    # the forward's segment states, handed to the backward, give the same
    # gradients bit for bit as the backward recomputing them
    B, H, N, D = shape
    tq, tk, tv, tg, tl, S0, tS0 = bwd_case(B, H, N, D, seed=N + 11, with_state=with_state)
    saved = torch.empty(la.retention_saved_bytes(B, H, N, D, D), dtype=torch.uint8, device=DEV)
    y = la.retention_forward(tq, tk, tv, tl, S0=tS0, saved=saved)
    with_saved = la.retention_backward(tq, tk, tv, tl, tg, S0=tS0, saved=saved)
    recomputed = la.retention_backward(tq, tk, tv, tl, tg, S0=tS0)
    torch.cuda.synchronize()
    for a, b in zip(with_saved, recomputed):
        assert torch.equal(a, b)
    check(y, ret.recurrent(f64(tq), f64(tk), f64(tv), f64(tl), S0)[0], f"forward keeping states {shape}")


def test_retention_saved_too_small_is_rejected():
    tq, tk, tv, tg, tl, _, _ = bwd_case(1, 2, 3000, 64, seed=5)
    n = la.retention_saved_bytes(1, 2, 3000, 64, 64)
    short = torch.empty(n - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(la.LinAttnError, match="INVALID"):
        la.retention_forward(tq, tk, tv, tl, saved=short)
    with pytest.raises(la.LinAttnError, match="INVALID"):
        la.retention_backward(tq, tk, tv, tl, tg, saved=short)


def test_retention_fwdbwd_workload():
    # The benchmark's retention step at full size (B=8, H=16, N=8192,
    # D=M=64, bf16, gates gamma_t ~ U(0.6, 1), automatic plan: 4 segments,
    # the forward keeping its segment states for the backward), checked on 4
    # heads spread over b and h against the oracle's recurrence and its
    # backward.
    from workloads import device_inputs

    B, H, N, D = 8, 16, 8192, 64
    tq, tk, tv, tg = device_inputs(B, H, N, D, D, "bf16", seed=2, scale=1.0 / np.sqrt(D))
    gen = torch.Generator(device=DEV).manual_seed(3)
    tl = torch.log(torch.rand(B, H, N, device=DEV, generator=gen) * 0.4 + 0.6)
    assert la.resolve_plan("retention_backward", B, H, N, D, D, True, "bf16")["segments"] == 4
    saved = torch.empty(la.retention_saved_bytes(B, H, N, D, D), dtype=torch.uint8, device=DEV)
    y = la.retention_forward(tq, tk, tv, tl, saved=saved)
    got = la.retention_backward(tq, tk, tv, tl, tg, saved=saved)
    torch.cuda.synchronize()
    heads = [(0, 0), (2, 9), (5, 4), (7, 15)]
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]

    def pick(t):
        return f64(t[bi, hi])[None]

    q64, k64, v64, g64, l64 = (pick(t) for t in (tq, tk, tv, tg, tl))
    say(f"retention workload: {B}x{H}x{N} D={D}, heads {heads}")
    check(y[bi, hi][None], ret.recurrent(q64, k64, v64, l64)[0], "workload forward")
    want = ret.backward(q64, k64, v64, l64, g64)
    check_grads([t[bi, hi][None] for t in got], want, "workload backward", q=tq[bi, hi][None])
    del tq, tk, tv, tg, tl, saved, y, got
    torch.cuda.empty_cache()
