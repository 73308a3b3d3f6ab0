"""la_forward_noalloc: the forward whose segment records live in the
library's static device scratch instead of a caller workspace.  Checked
through the C ABI against la_forward with a workspace (same plan and kernels:
bit for bit), on two calls in a row, the second smaller, so that the second
reuses the scratch the first left behind."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import kernelized_causal_attention_amd as la
import oracle
from kernelized_causal_attention_amd import _native
from workloads import numpy_inputs, rel_l2, to_torch

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCRATCH_BYTES = 64 << 20


def say(*a):
    print("[noalloc]", *a, file=sys.stderr, flush=True)


def call_noalloc(q, k, v, causal, with_den=True):
    lib = _native.load()
    B, H, N, D = q.shape
    M = v.shape[3]
    out = torch.full_like(v, float("nan"))
    den = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV) if with_den else None
    dt = _native.LA_F32 if q.dtype == torch.float32 else _native.LA_BF16
    st = lib.la_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, D, M,
                                int(causal), dt, None if den is None else den.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.la_last_error()
    return out, den


def call_with_workspace(q, k, v, causal):
    lib = _native.load()
    B, H, N, D = q.shape
    M = v.shape[3]
    dt = _native.LA_F32 if q.dtype == torch.float32 else _native.LA_BF16
    need = lib.la_workspace_bytes(0, B, H, N, D, M, int(causal), dt)
    assert 0 < need <= SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(v)
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    st = lib.la_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, D, M, int(causal), dt,
                        den.data_ptr(), ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.la_last_error()
    return out, den


# (first call, second smaller call): MFMA bf16 at D = 64 and 128, the fp32
# MFMA path, generic kernels (D != M); causal calls with several segments
# (records in the scratch) and non-causal ones (records and totals)
CASES = [
    ((2, 4, 3000, 64, 64, "bf16"), (1, 2, 700, 64, 64, "bf16")),
    ((1, 2, 4100, 128, 128, "bf16"), (1, 1, 1500, 128, 128, "bf16")),
    ((2, 2, 2500, 64, 64, "f32"), (1, 3, 900, 64, 64, "f32")),
    ((2, 3, 1000, 32, 16, "f32"), (1, 2, 333, 32, 16, "f32")),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_forward_matches_workspace_forward(first, second, causal):
    for n, (B, H, N, D, M, dtype) in enumerate((first, second)):
        say(f"call {n + 1}: B={B} H={H} N={N} D={D} M={M} {dtype} causal={causal}")
        q, k, v, _ = numpy_inputs(B, H, N, D, M, seed=N + D + n, scale=1.0 / np.sqrt(D), with_dout=False)
        tq, tk, tv = (to_torch(x, dtype, DEV) for x in (q, k, v))
        out, den = call_noalloc(tq, tk, tv, causal)
        ref_out, ref_den = call_with_workspace(tq, tk, tv, causal)
        torch.cuda.synchronize()
        for name, a, b in (("out", out, ref_out), ("den", den, ref_den)):
            if not torch.equal(a, b):
                bad = (a != b).reshape(-1, a.shape[-1]).any(dim=-1) if a.dim() == 4 else (a != b).reshape(-1)
                rows = torch.nonzero(bad).flatten().tolist()
                pytest.fail(f"{name} differs from la_forward's in {len(rows)} rows (flat (b, h, n) indices "
                            f"{rows[:8]}; N = {N}); max |diff| {(a.float() - b.float()).abs().nan_to_num(1e30).max():.3e}")
        # and the oracle, on the exact inputs
        o64, d64 = oracle.forward_recurrent(*(t.double().cpu().numpy() for t in (tq, tk, tv)), causal)[:2]
        e = rel_l2(out.double().cpu().numpy(), o64)
        say(f"  bit-identical to la_forward; vs oracle {e:.2e}")
        assert e < (1e-4 if dtype == "f32" else 2e-2)


def test_noalloc_rejects_calls_beyond_the_scratch():
    # non-causal with many heads needs one record per head and segment plus
    # the totals: more than 64 MiB at D = M = 128 -> refused before any launch
    lib = _native.load()
    B, H, N, D = 4, 256, 64, 128
    need = lib.la_workspace_bytes(0, B, H, N, D, D, 0, _native.LA_BF16)
    assert need > SCRATCH_BYTES
    t = torch.zeros((B, H, N, D), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(t)
    st = lib.la_forward_noalloc(t.data_ptr(), t.data_ptr(), t.data_ptr(), out.data_ptr(), B, H, N, D, D, 0,
                                _native.LA_BF16, None, torch.cuda.current_stream().cuda_stream)
    assert st == _native.LA_ERR_UNSUPPORTED and b"static scratch" in lib.la_last_error()


def test_noalloc_binding():
    q, k, v, _ = numpy_inputs(1, 2, 1000, 64, 64, seed=3, scale=0.125, with_dout=False)
    tq, tk, tv = (to_torch(x, "bf16", DEV) for x in (q, k, v))
    out = torch.empty_like(tv)
    la.forward_noalloc(tq, tk, tv, out=out)
    ref = la.forward(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
