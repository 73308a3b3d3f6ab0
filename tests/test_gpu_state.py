"""GPU parity of the state-carrying calls (la_forward_state, la_backward_state)
against the fp64 oracle, through the C ABI.

A state (S0, Z0) left by earlier tokens ("[Paper walkthrough] Transformers
are RNNs", section 4; "The deep link between Transformer and RNN", section
4.2) enters every row; the oracle's forward_quadratic / backward_state with
S0, Z0 are pinned by the continuation property and finite differences.  The
states used here are those of real prefixes (computed by the oracle in fp64
from the same rounded tokens), so their scale is a real session's.
"""

import sys

import numpy as np
import pytest
import torch

import kernelized_causal_attention_amd as la
import oracle
from workloads import numpy_inputs, rel_l2, to_torch

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda"


def say(*a):
    print("[state]", *a, file=sys.stderr, flush=True)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def case(B, H, N, D, M, dtype, seed, prefix, shift=0.0):
    """Device tensors for N tokens, and the fp64 state of `prefix` earlier
    tokens of the same sequence (zero state when prefix == 0).  shift moves
    q and k (unscaled N(0, 1) then) so that phi = e^x is small in every
    feature."""
    q, k, v, g = numpy_inputs(B, H, N + prefix, D, M, seed=seed, scale=1.0 / np.sqrt(D))
    if shift:
        q, k = q * np.sqrt(D) + shift, k * np.sqrt(D) + shift
    tq, tk, tv, tg = (to_torch(x[..., prefix:, :], dtype, DEV) for x in (q, k, v, g))
    if prefix:
        pk, pv = (f64(to_torch(x[..., :prefix, :], dtype, DEV)) for x in (k, v))
        S0, Z0 = oracle.prefix_state(pk, pv)
    else:
        S0, Z0 = np.zeros((B, H, D, M)), np.zeros((B, H, D))
    return tq, tk, tv, tg, S0, Z0


STATE_CASES = [
    # (B, H, N, D, M, dtype, prefix, shift): generic fp32 (D != M), MFMA bf16
    # D = 64 / 128; N spans several chunks and segments, with a ragged tail;
    # shifted features (phi << 1 everywhere, the per-feature split's mu = 0)
    (2, 2, 333, 32, 16, "f32", 100, 0.0),
    (2, 2, 700, 64, 64, "bf16", 300, 0.0),
    (1, 2, 1100, 128, 128, "bf16", 257, 0.0),
    (1, 1, 1, 64, 64, "bf16", 50, 0.0),
    (2, 1, 90, 64, 64, "bf16", 0, 0.0),
    (1, 2, 700, 64, 64, "bf16", 300, -3.0),
    (1, 1, 1100, 128, 128, "bf16", 257, -3.0),
    # ten segments: the scan from (S0, Z0) reads a full batch of eight
    # records and a partial one
    (1, 1, 2500, 64, 64, "bf16", 200, 0.0),
]


@pytest.mark.parametrize("B,H,N,D,M,dtype,prefix,shift", STATE_CASES)
def test_forward_state_matches_oracle(B, H, N, D, M, dtype, prefix, shift):
    tq, tk, tv, _, S0, Z0 = case(B, H, N, D, M, dtype, seed=N + D + prefix, prefix=prefix, shift=shift)
    tS0 = torch.tensor(S0, dtype=torch.float32, device=DEV)
    tZ0 = torch.tensor(Z0, dtype=torch.float32, device=DEV)
    out, S, Z, den = la.forward_state(tq, tk, tv, tS0, tZ0, return_den=True)
    torch.cuda.synchronize()
    q64, k64, v64 = f64(tq), f64(tk), f64(tv)
    ref, rden, rS, rZ = oracle.forward_recurrent(q64, k64, v64, True, S0, Z0)
    e = {"out": rel_l2(f64(out), ref), "den": rel_l2(f64(den), rden), "S": rel_l2(f64(S), rS),
         "Z": rel_l2(f64(Z), rZ)}
    say(f"forward_state {(B, H, N, D, M)} {dtype} prefix={prefix} shift={shift} " + " ".join(f"{n}={x:.2e}" for n, x in e.items()))
    for n, x in e.items():
        assert x < TOL[dtype], (n, x)
    # the final state comes from the fp32 segment sums (elu carried as bf16 on
    # the MFMA path): far inside the tolerance
    assert e["S"] < (1e-5 if dtype == "f32" else 2e-3)
    assert e["Z"] < (1e-5 if dtype == "f32" else 2e-3)


@pytest.mark.parametrize("B,H,N,D,M,dtype,prefix,shift", STATE_CASES)
def test_backward_state_matches_oracle(B, H, N, D, M, dtype, prefix, shift):
    tq, tk, tv, tg, S0, Z0 = case(B, H, N, D, M, dtype, seed=N + D + prefix + 1, prefix=prefix, shift=shift)
    tS0 = torch.tensor(S0, dtype=torch.float32, device=DEV)
    tZ0 = torch.tensor(Z0, dtype=torch.float32, device=DEV)
    out, _, _ = la.forward_state(tq, tk, tv, tS0, tZ0)
    dq, dk, dv, dS0, dZ0 = la.backward_state(tq, tk, tv, out, tg, tS0, tZ0)
    torch.cuda.synchronize()
    rq, rk, rv, rS, rZ, _, _ = oracle.backward_state(f64(tq), f64(tk), f64(tv), f64(tg), S0, Z0, True)
    scale = np.linalg.norm(rv)

    def err(x, r):
        nr = np.linalg.norm(r)
        # dq, dk vanish identically only for one token with no carried state
        return float(np.linalg.norm(f64(x) - r) / (nr if nr > 1e-9 * scale else 1e-2 * scale))

    e = {n: err(x, r) for n, x, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv), ("dS0", dS0, rS),
                                     ("dZ0", dZ0, rZ))}
    say(f"backward_state {(B, H, N, D, M)} {dtype} prefix={prefix} shift={shift} " + " ".join(f"{n}={x:.2e}" for n, x in e.items()))
    for n, x in e.items():
        assert x < TOL[dtype], (n, x)
    if dtype == "bf16":
        # within 4x of the bf16 rounding of the exact gradients (5e-3 where
        # that vanishes), as for the plain backward
        for n, r in (("dq", rq), ("dk", rk), ("dv", rv)):
            e_round = err(torch.from_numpy(r).float().to(torch.bfloat16), r)
            assert e[n] < max(4.0 * e_round, 5e-3), (n, e[n], e_round)


@pytest.mark.parametrize("dtype,D", [("f32", 32), ("bf16", 64)])
def test_state_continues_the_sequence(dtype, D):
    # forward over all tokens == forward over a prefix, then forward_state
    # over the rest from the prefix's state (state handed across calls)
    B, H, N, a = 2, 2, 900, 377
    q, k, v, _ = numpy_inputs(B, H, N, D, D, seed=D + 5, scale=1.0 / np.sqrt(D))
    tq, tk, tv = (to_torch(x, dtype, DEV) for x in (q, k, v))
    full = la.forward(tq, tk, tv)
    o1, S1, Z1 = la.forward_state(tq[:, :, :a].contiguous(), tk[:, :, :a].contiguous(), tv[:, :, :a].contiguous())
    o2, S2, Z2 = la.forward_state(tq[:, :, a:].contiguous(), tk[:, :, a:].contiguous(), tv[:, :, a:].contiguous(),
                                  S1, Z1)
    Sf, Zf = la.prefix_state(tk, tv)
    torch.cuda.synchronize()
    ref = oracle.forward_recurrent(f64(tq), f64(tk), f64(tv), True)[0]
    both = torch.cat([o1, o2], dim=2)
    e_split = rel_l2(f64(both), ref)
    e_full = rel_l2(f64(full), ref)
    say(f"continuation {dtype} D={D}: split {e_split:.2e}, one call {e_full:.2e}")
    assert e_split < TOL[dtype] and e_full < TOL[dtype]
    # the split answer is as good as the single call's
    assert e_split < 1.5 * e_full + (1e-6 if dtype == "f32" else 1e-4)
    assert rel_l2(f64(S2), f64(Sf)) < (1e-5 if dtype == "f32" else 1e-3)
    assert rel_l2(f64(Z2), f64(Zf)) < (1e-5 if dtype == "f32" else 1e-3)


def test_state_updated_in_place_and_decode_handoff():
    # prefill 512 tokens into a session state, then 64 decode steps and a
    # 64-token multi-token step, all updating the same S, Z in place; the
    # outputs must match one causal pass over all 640 tokens.
    B, H, D = 2, 4, 64
    q, k, v, _ = numpy_inputs(B, H, 640, D, D, seed=77, scale=1.0 / np.sqrt(D))
    tq, tk, tv = (to_torch(x, "f32", DEV) for x in (q, k, v))
    S = torch.zeros(B, H, D, D, device=DEV)
    Z = torch.zeros(B, H, D, device=DEV)
    o_pre, S_r, Z_r = la.forward_state(tq[:, :, :512].contiguous(), tk[:, :, :512].contiguous(),
                                       tv[:, :, :512].contiguous(), S, Z, S_out=S, Z_out=Z)
    assert S_r.data_ptr() == S.data_ptr() and Z_r.data_ptr() == Z.data_ptr()
    outs = []
    for t in range(512, 576):
        outs.append(la.decode_step(S, Z, tq[:, :, t].contiguous(), tk[:, :, t].contiguous(), tv[:, :, t].contiguous()))
    o_multi, _, _ = la.forward_state(tq[:, :, 576:].contiguous(), tk[:, :, 576:].contiguous(),
                                     tv[:, :, 576:].contiguous(), S, Z, S_out=S, Z_out=Z)
    full = la.forward(tq, tk, tv)
    torch.cuda.synchronize()
    got = torch.cat([o_pre, torch.stack(outs, dim=2), o_multi], dim=2)
    ref = oracle.forward_recurrent(f64(tq), f64(tk), f64(tv), True)
    e_got = rel_l2(f64(got), ref[0])
    say(f"session: prefill + 64 decode steps + 64-token step {e_got:.2e}")
    assert e_got < TOL["f32"]
    assert rel_l2(f64(full), ref[0]) < TOL["f32"]
    assert rel_l2(f64(S), ref[2]) < 1e-5 and rel_l2(f64(Z), ref[3]) < 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,one_segment", [(2000, False), (200, True)])
def test_forward_state_without_state_outputs(dtype, N, one_segment):
    # la_forward_state with S_out = Z_out = NULL: the segment pass then skips
    # the last segment (its aggregate would only feed the total), and with a
    # single segment it is not launched at all (the scan writes S0, Z0 into
    # the record); the output must equal the call that also returns the
    # state, bit for bit
    B, H, D, M = 2, 3, 64, 64
    tq, tk, tv, _, S0, Z0 = case(B, H, N, D, M, dtype, seed=9, prefix=100)
    tS0 = torch.tensor(S0, dtype=torch.float32, device=DEV)
    tZ0 = torch.tensor(Z0, dtype=torch.float32, device=DEV)
    assert (la.resolve_plan("forward_state", B, H, N, D, M, True, dtype)["segments"] == 1) == one_segment
    want, _, _ = la.forward_state(tq, tk, tv, tS0, tZ0)
    lib = la._native.load()
    out = torch.empty_like(tv)
    nws = la.workspace_bytes("forward_state", B, H, N, D, M, True, dtype)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
    dt = {"f32": la._native.LA_F32, "bf16": la._native.LA_BF16}[dtype]
    st = lib.la_forward_state(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), B, H, N, D, M, dt,
                              tS0.data_ptr(), tZ0.data_ptr(), None, None, None, ws.data_ptr(), nws,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0, lib.la_last_error()
    assert torch.equal(out, want)


def test_state_arguments_are_validated():
    tq, tk, tv, _, S0, Z0 = case(1, 1, 64, 16, 16, "f32", seed=1, prefix=10)
    tS0 = torch.tensor(S0, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        la.forward_state(tq, tk, tv, tS0, None)
    lib = la._native.load()
    out = torch.empty_like(tv)
    # S0 without Z0 at the C ABI
    st = lib.la_forward_state(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), 1, 1, 64, 16, 16, 0,
                              tS0.data_ptr(), None, None, None, None, None, 0, None)
    assert st == la._native.LA_ERR_INVALID
    # a state output overlapping an input
    Z = torch.zeros(1, 1, 16, device=DEV)
    st = lib.la_forward_state(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), 1, 1, 64, 16, 16, 0,
                              None, None, tq.data_ptr(), Z.data_ptr(), None, None, 0, None)
    assert st == la._native.LA_ERR_INVALID and b"overlaps" in lib.la_last_error()
