"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds the workload shapes and the random-number recipes only; it
contains none of the method's arithmetic, and neither the oracle nor the HIP
binding imports it.  Callers pass the arrays it returns to both sides.

Recipe: ``numpy.random.default_rng(seed)``, draw order Q, K, V, dout, each a
float64 standard normal of the full C-ordered [B, H, N, feature] shape; Q, K
and V are scaled by 1/sqrt(D) where the workload says so (dout never is),
then rounded to the working dtype (float64 -> float32 -> bfloat16, round to
nearest even).  Device-side generation (for the multi-GB shapes) uses a
``torch.Generator`` on the GPU with the same order and scaling; the exact
tensors it produced are what any host-side check reads back.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    M: int
    dtype: str  # "f32" or "bf16"
    scaled: bool  # Q, K, V ~ N(0,1)/sqrt(D) when True, N(0,1) otherwise
    causal: bool = True
    prefix: int = 0  # decode only: tokens folded into the initial state
    steps: int = 0  # decode only: consecutive decode steps
    what: str = ""


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, 1, 64, 16, 16, "f32", False,
        what="tiny check, causal and non-causal forward plus backward, seed 0",
    ),
    "fwd_f32": Workload(
        "fwd_f32", 4, 8, 2048, 64, 64, "f32", True,
        what="causal forward, fp32",
    ),
    "fwdbwd_bf16": Workload(
        "fwdbwd_bf16", 8, 16, 8192, 64, 64, "bf16", True,
        what="causal forward+backward, bf16 inputs / fp32 accumulate",
    ),
    "long_bf16": Workload(
        "long_bf16", 1, 16, 65536, 128, 128, "bf16", True,
        what="long-sequence causal forward, bf16, 128x128 state per head",
    ),
    "decode_f32": Workload(
        "decode_f32", 256, 32, 0, 128, 128, "f32", True, prefix=512, steps=1024,
        what="batched RNN decode, fp32 state, 512-token prefix then 1024 steps",
    ),
}


def _scale(w: Workload) -> float:
    return 1.0 / math.sqrt(w.D) if w.scaled else 1.0


def numpy_inputs(B, H, N, D, M, seed=0, scale=1.0, with_dout=True):
    """float64 arrays q, k [B,H,N,D], v [B,H,N,M], dout [B,H,N,M] (or None)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, D)) * scale
    k = rng.standard_normal((B, H, N, D)) * scale
    v = rng.standard_normal((B, H, N, M)) * scale
    dout = rng.standard_normal((B, H, N, M)) if with_dout else None
    return q, k, v, dout


def to_torch(x, dtype: str, device="cpu"):
    """Round a float64 array to the working dtype as a torch tensor."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t.to(device)


def torch_dtype(dtype: str):
    import torch

    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def device_inputs(B, H, N, D, M, dtype: str, seed=0, scale=1.0, device="cuda",
                  with_dout=True, generator: Optional[object] = None):
    """Same recipe drawn on the device (for shapes too large for the host)."""
    import torch

    g = generator
    if g is None:
        g = torch.Generator(device=device)
        g.manual_seed(seed)
    td = torch_dtype(dtype)

    def draw(shape, s):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if s != 1.0:
            x.mul_(s)
        return x.to(td)

    q = draw((B, H, N, D), scale)
    k = draw((B, H, N, D), scale)
    v = draw((B, H, N, M), scale)
    dout = draw((B, H, N, M), 1.0) if with_dout else None
    return q, k, v, dout


def workload_inputs(w: Workload, seed=0, device="cpu"):
    """q, k, v, dout for a forward/backward workload as torch tensors.

    Host generation (numpy) for device="cpu"; device generation otherwise.
    """
    s = _scale(w)
    if device == "cpu":
        q, k, v, g = numpy_inputs(w.B, w.H, w.N, w.D, w.M, seed, s)
        return tuple(to_torch(x, w.dtype) for x in (q, k, v)) + (to_torch(g, "f32"),)
    return device_inputs(w.B, w.H, w.N, w.D, w.M, w.dtype, seed, s, device)


def decode_inputs(w: Workload, seed=0, device="cuda"):
    """Prefix q, k, v [B,H,prefix,D] and step q, k, v [steps,B,H,D] (fp32)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    s = _scale(w)

    def draw(shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(s)

    pq = draw((w.B, w.H, w.prefix, w.D))
    pk = draw((w.B, w.H, w.prefix, w.D))
    pv = draw((w.B, w.H, w.prefix, w.M))
    sq = draw((w.steps, w.B, w.H, w.D))
    sk = draw((w.steps, w.B, w.H, w.D))
    sv = draw((w.steps, w.B, w.H, w.M))
    return (pq, pk, pv), (sq, sk, sv)


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over all elements, in float64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / np.linalg.norm(ref.ravel()))


def null_model(v, causal=True):
    """Running mean of V (ignores Q and K): the guard a kernel must beat."""
    v = np.asarray(v, dtype=np.float64)
    if not causal:
        return np.broadcast_to(v.mean(axis=-2, keepdims=True), v.shape)
    n = v.shape[-2]
    cnt = np.arange(1, n + 1, dtype=np.float64)[:, None]
    return np.cumsum(v, axis=-2) / cnt
