"""The C-ABI calls under HIP graph capture: a captured forward + backward
step and a captured run of decode steps, replayed several times with the
program's own eager work (new inputs copied in, synchronisations) between
the replays, each replay checked against the same calls run eagerly on the
same inputs.

The library allocates nothing, clears nothing with memset and synchronises
nothing inside its calls, and every kernel sums in a fixed order, so a replay
must reproduce the eager results bit for bit.
"""

import sys

import numpy as np
import pytest
import torch

import kernelized_causal_attention_amd as la
from workloads import device_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print("[graph]", *a, file=sys.stderr, flush=True)


def _step(q, k, v, g, out, den, ws_f, ws_b, saved):
    la.forward(q, k, v, causal=True, out=out, den=den, return_den=True, workspace=ws_f, saved=saved)
    return la.backward(q, k, v, out, g, den=den, causal=True, workspace=ws_b, saved=saved)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_graph_forward_backward_replays_match_eager(dtype, D):
    B, H, N = 2, 3, 1000
    args = (B, H, N, D, D, True, dtype)
    q, k, v, g = device_inputs(B, H, N, D, D, dtype, seed=0, scale=1.0 / np.sqrt(D))
    out, den = torch.empty_like(v), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws_f = torch.empty(max(1, la.workspace_bytes("forward", *args)), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(1, la.workspace_bytes("backward", *args)), dtype=torch.uint8, device="cuda")
    # fp32 runs the forward on MFMA kernels and the backward on the generic
    # ones, whose segment plans differ, so only bf16 hands states over
    ns = la.saved_bytes(*args) if dtype == "bf16" else 0
    saved = torch.empty(ns, dtype=torch.uint8, device="cuda") if ns else None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        _step(q, k, v, g, out, den, ws_f, ws_b, saved)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gq, gk, gv = _step(q, k, v, g, out, den, ws_f, ws_b, saved)
    for seed in (1, 2, 3):
        nq, nk, nv, ng = device_inputs(B, H, N, D, D, dtype, seed=seed, scale=1.0 / np.sqrt(D))
        for dst, src in ((q, nq), (k, nk), (v, nv), (g, ng)):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (out, den, gq, gk, gv)]
        eo = torch.empty_like(out)
        ed = torch.empty_like(den)
        edq, edk, edv = _step(nq, nk, nv, ng, eo, ed, ws_f, ws_b, saved)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "den", "dq", "dk", "dv"), got, (eo, ed, edq, edk, edv)):
            assert torch.equal(a, b), (dtype, D, seed, name, (a.float() - b.float()).abs().max().item())
        say(f"{dtype} D={D} replay seed {seed}: out, den, dq, dk, dv bit-identical to eager")


def test_graph_decode_steps_replay_match_eager():
    B, H, D, steps = 8, 4, 128, 8
    gen = torch.Generator(device="cuda").manual_seed(5)
    S0 = torch.randn(B, H, D, D, device="cuda", generator=gen) * 0.1
    Z0 = torch.rand(B, H, D, device="cuda", generator=gen) * 50 + 10
    q, k, v = (torch.randn(steps, B, H, D, device="cuda", generator=gen) * D ** -0.5 for _ in range(3))
    S, Z = S0.clone(), Z0.clone()
    outs = torch.empty(steps, B, H, D, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        la.decode_step(S, Z, q[0], k[0], v[0], out=outs[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(steps):
            la.decode_step(S, Z, q[t], k[t], v[t], out=outs[t])
    for rep in range(3):
        S.copy_(S0)
        Z.copy_(Z0)
        graph.replay()
        torch.cuda.synchronize()
        rS, rZ = S0.clone(), Z0.clone()
        ref = torch.empty_like(outs)
        for t in range(steps):
            la.decode_step(rS, rZ, q[t], k[t], v[t], out=ref[t])
        torch.cuda.synchronize()
        assert torch.equal(outs, ref) and torch.equal(S, rS) and torch.equal(Z, rZ), rep
        say(f"decode replay {rep}: {steps} steps bit-identical to eager")
