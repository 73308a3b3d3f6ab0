"""MI355X-native causal linear attention (phi = elu + 1), "Transformers are RNNs".

Thin Python binding over the C ABI of ``_lib/liblinattn.so`` (hand-written HIP
kernels for gfx950).  The functions here only check tensor metadata, allocate
outputs and workspace through torch and pass raw device pointers plus the
current HIP stream; every step of the computation runs in the library's
kernels.  Names follow the C ABI: ``forward`` -> ``la_forward``,
``backward`` -> ``la_backward``, ``decode_step`` -> ``la_decode_step``,
``prefix_state`` -> ``la_prefix_state``.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

from . import _native
from ._native import LinAttnError, la_plan  # noqa: F401

__all__ = [
    "forward", "forward_noalloc", "backward", "forward_state", "backward_state", "decode_step", "prefix_state", "workspace_bytes",
    "saved_bytes", "resolve_plan", "retention_forward", "retention_backward", "retention_decode_step",
    "retention_saved_bytes", "poly_forward", "poly_backward", "poly_prefix_state", "poly_decode_step",
    "softmax_forward", "softmax_decode_step",
    "LinAttnError", "library_path", "version", "profile_enable", "profile_report",
]

library_path = _native.LIB_PATH


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return _native.LA_F32
    if t.dtype == torch.bfloat16:
        return _native.LA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _plan(plan) -> Optional[la_plan]:
    if plan is None:
        return None
    if isinstance(plan, la_plan):
        return plan
    return la_plan(int(plan.get("chunk", 0)), int(plan.get("segments", 0)), int(plan.get("kernel", 0)))


def _plan_ref(p: Optional[la_plan]):
    return None if p is None else ctypes.byref(p)


def version() -> int:
    return _native.load().la_version()


def profile_enable(on: bool = True, only=None) -> None:
    """Start (clearing old records) or stop per-kernel HIP-event timing;
    `only` restricts it to the named kernels (list or comma-separated)."""
    lib = _native.load()
    names = "" if only is None else (only if isinstance(only, str) else ",".join(only))
    _native.check(lib.la_profile_select(names.encode()))
    _native.check(lib.la_profile_enable(int(bool(on))))


def profile_report() -> dict:
    """{kernel name: (launches, total ms)} since profile_enable(True); clears."""
    buf = ctypes.create_string_buffer(1 << 16)
    _native.check(_native.load().la_profile_report(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split()
        out[name] = (int(n), float(ms))
    return out


_OPS = {"forward": _native.LA_OP_FORWARD, "backward": _native.LA_OP_BACKWARD,
        "prefix_state": _native.LA_OP_PREFIX_STATE, "decode": _native.LA_OP_DECODE,
        "forward_state": _native.LA_OP_FORWARD_STATE, "backward_state": _native.LA_OP_BACKWARD_STATE,
        "retention_forward": _native.LA_OP_RETENTION_FORWARD,
        "retention_backward": _native.LA_OP_RETENTION_BACKWARD, "poly_backward": _native.LA_OP_POLY_BACKWARD}


def workspace_bytes(op: str, B, H, N, D, M, causal=True, dtype="f32", plan=None) -> int:
    dt = {"f32": _native.LA_F32, "bf16": _native.LA_BF16}[dtype]
    p = _plan(plan)
    return int(_native.load().la_workspace_bytes_ex(_OPS[op], B, H, N, D, M, int(bool(causal)), dt, _plan_ref(p)))


def resolve_plan(op: str, B, H, N, D, M, causal=True, dtype="f32", plan=None) -> dict:
    dt = {"f32": _native.LA_F32, "bf16": _native.LA_BF16}[dtype]
    out = la_plan()
    _native.check(_native.load().la_resolve_plan(_OPS[op], B, H, N, D, M, int(bool(causal)), dt,
                                                 _plan_ref(_plan(plan)), ctypes.byref(out)))
    return {"chunk": out.chunk, "segments": out.segments, "kernel": out.kernel}


def _workspace(nbytes: int, device):
    torch = _torch()
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def saved_bytes(B, H, N, D, M, causal=True, dtype="f32", plan=None) -> int:
    dt = {"f32": _native.LA_F32, "bf16": _native.LA_BF16}[dtype]
    return int(_native.load().la_saved_bytes(B, H, N, D, M, int(bool(causal)), dt, _plan_ref(_plan(plan))))


def forward(q, k, v, causal: bool = True, return_den: bool = False, plan=None, stream=None,
            out=None, den=None, workspace=None, saved=None):
    """V' = phi(Q) S / phi(Q) Z (causal) or phi(Q)(phi(K)^T V) normalised.

    q, k: [B,H,N,D]; v: [B,H,N,M]; float32 or bfloat16 (all the same).
    Returns out [B,H,N,M] (and den [B,H,N] fp32 when return_den).  When
    `saved` is a GPU tensor of at least saved_bytes(...) bytes, the prefix
    states are also kept there for backward(saved=...).
    """
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, H, N, D = q.shape
    M = v.shape[3]
    dt = _dtype_code(q)
    p = _plan(plan)
    lib = _native.load()
    if out is None:
        out = torch.empty((B, H, N, M), dtype=q.dtype, device=q.device)
    if return_den and den is None:
        den = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    need = int(lib.la_workspace_bytes_ex(_native.LA_OP_FORWARD, B, H, N, D, M, int(bool(causal)), dt, _plan_ref(p)))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    ssz = 0 if saved is None else _dev(saved, "saved").numel() * saved.element_size()
    _native.check(lib.la_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, D, M,
                                    int(bool(causal)), dt, _ptr(den), _ptr(saved), ssz, _ptr(ws), wsz,
                                    _stream(stream), _plan_ref(p)))
    return (out, den) if return_den else out


def forward_noalloc(q, k, v, causal: bool = True, out=None, den=None, stream=None):
    """forward() through la_forward_noalloc: the library's static device
    scratch replaces the workspace.  `out` (and `den`, when the row
    denominators are wanted) must be given: nothing is allocated, here or in
    the library.  Calls that overlap on one GPU share the scratch and race."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if t is None:
            raise ValueError(f"{n} must be given")
        _dev(t, n)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3] or out.shape != v.shape:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)} out{tuple(out.shape)}")
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise TypeError("q, k, v, out must share one dtype")
    B, H, N, D = q.shape
    M = v.shape[3]
    if den is not None:
        _dev(den, "den")
    _native.check(_native.load().la_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B,
                                                    H, N, D, M, int(bool(causal)), _dtype_code(q), _ptr(den),
                                                    _stream(stream)))
    return out


def backward(q, k, v, out, dout, den=None, causal: bool = True, plan=None, stream=None,
             workspace=None, saved=None) -> Tuple:
    """Gradients (dq, dk, dv) of sum(dout * out) w.r.t. the raw q, k, v.

    `saved`: the tensor forward(saved=...) filled for these inputs and the
    same plan; the prefix states are then read instead of recomputed."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _dev(t, n)
    B, H, N, D = q.shape
    M = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or out.shape != v.shape or dout.shape != v.shape:
        raise ValueError("shape mismatch")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise TypeError("q, k, v, out, dout must share one dtype")
    if den is not None:
        _dev(den, "den")
        if den.dtype != torch.float32 or tuple(den.shape) != (B, H, N):
            raise ValueError("den must be float32 [B,H,N]")
    dt = _dtype_code(q)
    p = _plan(plan)
    lib = _native.load()
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    need = int(lib.la_workspace_bytes_ex(_native.LA_OP_BACKWARD, B, H, N, D, M, int(bool(causal)), dt, _plan_ref(p)))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    ssz = 0 if saved is None else _dev(saved, "saved").numel() * saved.element_size()
    _native.check(lib.la_backward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                     _ptr(den), _ptr(saved), ssz, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                     B, H, N, D, M, int(bool(causal)), dt, _ptr(ws), wsz, _stream(stream),
                                     _plan_ref(p)))
    return dq, dk, dv


def _state_pair(S, Z, B, H, D, M, name):
    torch = _torch()
    if (S is None) != (Z is None):
        raise ValueError(f"{name}: give both S and Z, or neither")
    if S is None:
        return None, None
    for t, n in ((S, "S"), (Z, "Z")):
        _dev(t, f"{name} {n}")
        if t.dtype != torch.float32:
            raise TypeError(f"{name} {n} must be float32")
    if tuple(S.shape) != (B, H, D, M) or tuple(Z.shape) != (B, H, D):
        raise ValueError(f"{name}: S [B,H,D,M] and Z [B,H,D] expected")
    return S, Z


def forward_state(q, k, v, S0=None, Z0=None, out=None, S_out=None, Z_out=None, return_den=False, stream=None,
                  workspace=None):
    """Causal forward continuing from the state (S0, Z0) of earlier tokens
    (None: zero state).  Returns (out, S_N, Z_N) -- and den when return_den --
    where S_N, Z_N is the state after these tokens (written into S_out, Z_out
    when given; pass S_out=S0, Z_out=Z0 to update a session's state in
    place)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, H, N, D = q.shape
    M = v.shape[3]
    S0, Z0 = _state_pair(S0, Z0, B, H, D, M, "S0/Z0")
    if S_out is None:
        S_out = torch.empty((B, H, D, M), dtype=torch.float32, device=q.device)
        Z_out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    S_out, Z_out = _state_pair(S_out, Z_out, B, H, D, M, "S_out/Z_out")
    if out is None:
        out = torch.empty((B, H, N, M), dtype=q.dtype, device=q.device)
    den = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_den else None
    lib = _native.load()
    need = int(lib.la_workspace_bytes(_native.LA_OP_FORWARD_STATE, B, H, N, D, M, 1, _dtype_code(q)))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _native.check(lib.la_forward_state(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, D, M,
                                       _dtype_code(q), _ptr(S0), _ptr(Z0), _ptr(S_out), _ptr(Z_out), _ptr(den),
                                       _ptr(ws), wsz, _stream(stream)))
    return (out, S_out, Z_out, den) if return_den else (out, S_out, Z_out)


def backward_state(q, k, v, out, dout, S0=None, Z0=None, den=None, stream=None, workspace=None):
    """Gradients (dq, dk, dv, dS0, dZ0) of sum(dout * out) for forward_state
    from (S0, Z0) (None: zero state; dS0, dZ0 are still returned)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _dev(t, n)
    B, H, N, D = q.shape
    M = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or out.shape != v.shape or dout.shape != v.shape:
        raise ValueError("shape mismatch")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise TypeError("q, k, v, out, dout must share one dtype")
    S0, Z0 = _state_pair(S0, Z0, B, H, D, M, "S0/Z0")
    if den is not None:
        _dev(den, "den")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dS0 = torch.empty((B, H, D, M), dtype=torch.float32, device=q.device)
    dZ0 = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    lib = _native.load()
    need = int(lib.la_workspace_bytes(_native.LA_OP_BACKWARD_STATE, B, H, N, D, M, 1, _dtype_code(q)))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _native.check(lib.la_backward_state(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                        _ptr(den), _ptr(S0), _ptr(Z0), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                        dS0.data_ptr(), dZ0.data_ptr(), B, H, N, D, M, _dtype_code(q), _ptr(ws), wsz,
                                        _stream(stream)))
    return dq, dk, dv, dS0, dZ0


def retention_saved_bytes(B, H, N, D, M, dtype="bf16") -> int:
    """Bytes of retention_forward's `saved` record (0 when unsupported)."""
    dt = {"f32": _native.LA_F32, "bf16": _native.LA_BF16}[dtype]
    return int(_native.load().la_retention_saved_bytes(B, H, N, D, M, dt))


def retention_forward(q, k, v, log_gamma, S0=None, S_out=None, return_state=False, stream=None, workspace=None,
                      saved=None):
    """Decayed / gated linear attention: y_t = S_t^T q_t with
    S_t = gamma_t S_{t-1} + k_t v_t^T (log_gamma [B,H,N] fp32, <= 0; S0 the
    state carried in or None).  Returns y, and the final state too when
    return_state (written into S_out when given; S_out=S0 updates in place).
    `saved` (a device buffer of retention_saved_bytes()) keeps the segment
    states for retention_backward."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (log_gamma, "log_gamma")):
        _dev(t, n)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    B, H, N, D = q.shape
    M = v.shape[3]
    if log_gamma.dtype != torch.float32 or tuple(log_gamma.shape) != (B, H, N):
        raise ValueError("log_gamma must be float32 [B,H,N]")
    for t, n in ((S0, "S0"), (S_out, "S_out")):
        if t is not None:
            _dev(t, n)
            if t.dtype != torch.float32 or tuple(t.shape) != (B, H, D, M):
                raise ValueError(f"{n} must be float32 [B,H,D,M]")
    if return_state and S_out is None:
        S_out = torch.empty((B, H, D, M), dtype=torch.float32, device=q.device)
    y = torch.empty((B, H, N, M), dtype=q.dtype, device=q.device)
    lib = _native.load()
    need = int(lib.la_workspace_bytes(_native.LA_OP_RETENTION_FORWARD, B, H, N, D, M, 1, _dtype_code(q)))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    if saved is not None:
        _dev(saved, "saved")
    ssz = 0 if saved is None else saved.numel() * saved.element_size()
    _native.check(lib.la_retention_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_gamma.data_ptr(),
                                           y.data_ptr(), B, H, N, D, M, _dtype_code(q), _ptr(S0), _ptr(S_out),
                                           _ptr(saved), ssz, _ptr(ws), wsz, _stream(stream)))
    return (y, S_out) if return_state else y


def retention_backward(q, k, v, log_gamma, dy, S0=None, stream=None, workspace=None, saved=None):
    """Gradients (dq, dk, dv, dlog_gamma, dS0) of sum(dy * y) for
    retention_forward (dS0 is returned whether or not S0 was given).
    `saved`: the record retention_forward kept for the same inputs, or None."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (log_gamma, "log_gamma"), (dy, "dy")):
        _dev(t, n)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    B, H, N, D = q.shape
    M = v.shape[3]
    if dy.shape != v.shape or dy.dtype != q.dtype:
        raise ValueError("dy must match v")
    if log_gamma.dtype != torch.float32 or tuple(log_gamma.shape) != (B, H, N):
        raise ValueError("log_gamma must be float32 [B,H,N]")
    if S0 is not None:
        _dev(S0, "S0")
        if S0.dtype != torch.float32 or tuple(S0.shape) != (B, H, D, M):
            raise ValueError("S0 must be float32 [B,H,D,M]")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dlg = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dS0 = torch.empty((B, H, D, M), dtype=torch.float32, device=q.device)
    lib = _native.load()
    need = int(lib.la_workspace_bytes(_native.LA_OP_RETENTION_BACKWARD, B, H, N, D, M, 1, _dtype_code(q)))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    if saved is not None:
        _dev(saved, "saved")
    ssz = 0 if saved is None else saved.numel() * saved.element_size()
    _native.check(lib.la_retention_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_gamma.data_ptr(),
                                            dy.data_ptr(), _ptr(S0), _ptr(saved), ssz, dq.data_ptr(),
                                            dk.data_ptr(), dv.data_ptr(),
                                            dlg.data_ptr(), dS0.data_ptr(), B, H, N, D, M, _dtype_code(q), _ptr(ws),
                                            wsz, _stream(stream)))
    return dq, dk, dv, dlg, dS0


def retention_decode_step(S, q, k, v, log_gamma, out=None, stream=None):
    """One decayed recurrent step in place: S <- gamma S + k v^T, returns
    y = S^T q (q, k [B,H,D], v [B,H,M], log_gamma [B,H] fp32, S fp32
    [B,H,D,M])."""
    torch = _torch()
    for t, n in ((S, "S"), (q, "q"), (k, "k"), (v, "v"), (log_gamma, "log_gamma")):
        _dev(t, n)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    B, H, D = q.shape
    M = v.shape[2]
    if S.dtype != torch.float32 or tuple(S.shape) != (B, H, D, M):
        raise ValueError("S must be float32 [B,H,D,M]")
    if log_gamma.dtype != torch.float32 or tuple(log_gamma.shape) != (B, H):
        raise ValueError("log_gamma must be float32 [B,H]")
    y = out if out is not None else torch.empty((B, H, M), dtype=q.dtype, device=q.device)
    lib = _native.load()
    _native.check(lib.la_retention_decode_step(S.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               log_gamma.data_ptr(), y.data_ptr(), B, H, D, M, _dtype_code(q),
                                               _stream(stream)))
    return y


def poly_forward(q, k, v, causal=True, out=None, den=None, return_den=False, stream=None):
    """Degree-2 polynomial-kernel attention: out_i = sum_j (q_i.k_j)^2 v_j /
    sum_j (q_i.k_j)^2 over j <= i (causal) or all j (0 where every weight is
    0).  bf16, D = M in {64, 128}.  Returns out (and den when return_den)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    B, H, N, D = q.shape
    M = v.shape[3]
    if out is None:
        out = torch.empty((B, H, N, M), dtype=q.dtype, device=q.device)
    if return_den and den is None:
        den = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _native.check(_native.load().la_poly_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(den),
                                                 B, H, N, D, M, int(bool(causal)), _dtype_code(q), _stream(stream)))
    return (out, den) if return_den else out


def poly_backward(q, k, v, out, dout, den, causal=True, stream=None, workspace=None):
    """Gradients (dq, dk, dv) of sum(dout * out) for poly_forward, given its
    out and den."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"), (den, "den")):
        _dev(t, n)
    B, H, N, D = q.shape
    M = v.shape[3]
    if out.shape != v.shape or dout.shape != v.shape or tuple(den.shape) != (B, H, N) or den.dtype != torch.float32:
        raise ValueError("out, dout must match v; den must be float32 [B,H,N]")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    lib = _native.load()
    need = int(lib.la_workspace_bytes(_native.LA_OP_POLY_BACKWARD, B, H, N, D, M, int(bool(causal)), _dtype_code(q)))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _native.check(lib.la_poly_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                       den.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, D, M,
                                       int(bool(causal)), _dtype_code(q), _ptr(ws), wsz, _stream(stream)))
    return dq, dk, dv


def poly_prefix_state(k, v, stream=None):
    """(S, Z) of the polynomial map after the given tokens: S [B,H,D*D,M],
    Z [B,H,D*D] fp32 (bf16 k, v; D = M in {64, 128})."""
    torch = _torch()
    _dev(k, "k")
    _dev(v, "v")
    B, H, N, D = k.shape
    M = v.shape[3]
    S = torch.empty((B, H, D * D, M), dtype=torch.float32, device=k.device)
    Z = torch.empty((B, H, D * D), dtype=torch.float32, device=k.device)
    _native.check(_native.load().la_poly_prefix_state(k.data_ptr(), v.data_ptr(), S.data_ptr(), Z.data_ptr(), B, H, N,
                                                      D, M, _dtype_code(k), _stream(stream)))
    return S, Z


def poly_decode_step(S, Z, q, k, v, out=None, stream=None):
    """One polynomial-map recurrent step in place: S += phi(k) v^T,
    Z += phi(k); returns phi(q)^T S / phi(q)^T Z (q, k [B,H,D], v [B,H,M])."""
    torch = _torch()
    for t, n in ((S, "S"), (Z, "Z"), (q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    B, H, D = q.shape
    M = v.shape[2]
    if tuple(S.shape) != (B, H, D * D, M) or tuple(Z.shape) != (B, H, D * D):
        raise ValueError("S must be [B,H,D*D,M] and Z [B,H,D*D] (float32)")
    if out is None:
        out = torch.empty((B, H, M), dtype=q.dtype, device=q.device)
    _native.check(_native.load().la_poly_decode_step(S.data_ptr(), Z.data_ptr(), q.data_ptr(), k.data_ptr(),
                                                     v.data_ptr(), out.data_ptr(), B, H, D, M, _dtype_code(q),
                                                     _stream(stream)))
    return out


def softmax_forward(q, k, v, causal=True, out=None, lse=None, return_lse=False, stream=None):
    """Softmax attention softmax(q k^T / sqrt(D)) v, causal or not (bf16,
    D = M in {64, 128}).  Returns out (and lse when return_lse)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    B, H, N, D = q.shape
    M = v.shape[3]
    if out is None:
        out = torch.empty((B, H, N, M), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _native.check(_native.load().la_softmax_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                    _ptr(lse), B, H, N, D, M, int(bool(causal)), _dtype_code(q),
                                                    _stream(stream)))
    return (out, lse) if return_lse else out


def softmax_decode_step(k_cache, v_cache, L, q, k, v, out=None, stream=None):
    """One KV-cache step: writes (k, v) at position L of the caches
    ([B,H,capacity,D] / [B,H,capacity,M]) and returns the attention of q over
    positions 0..L.  The caller advances L."""
    torch = _torch()
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    B, H, cap, D = k_cache.shape
    M = v_cache.shape[3]
    if out is None:
        out = torch.empty((B, H, M), dtype=q.dtype, device=q.device)
    _native.check(_native.load().la_softmax_decode_step(k_cache.data_ptr(), v_cache.data_ptr(), q.data_ptr(),
                                                        k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, L, cap, D,
                                                        M, _dtype_code(q), _stream(stream)))
    return out


def decode_step(S, Z, q, k, v, out=None, stream=None):
    """One in-place RNN step: S += phi(k) v^T, Z += phi(k); returns
    out = phi(q)^T S / phi(q)^T Z.  S [B,H,D,M] fp32, Z [B,H,D] fp32,
    q, k [B,H,D], v [B,H,M] (float32 or bfloat16)."""
    torch = _torch()
    for t, n in ((S, "S"), (Z, "Z"), (q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if S.dtype != torch.float32 or Z.dtype != torch.float32:
        raise TypeError("S and Z are float32")
    B, H, D, M = S.shape
    if tuple(Z.shape) != (B, H, D) or tuple(q.shape) != (B, H, D) or k.shape != q.shape or tuple(v.shape) != (B, H, M):
        raise ValueError("shape mismatch")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, M), dtype=q.dtype, device=q.device)
    _native.check(_native.load().la_decode_step(S.data_ptr(), Z.data_ptr(), q.data_ptr(), k.data_ptr(),
                                                v.data_ptr(), out.data_ptr(), B, H, D, M, dt, _stream(stream)))
    return out


def prefix_state(k, v, S=None, Z=None, stream=None):
    """S = sum_j phi(K_j) V_j^T, Z = sum_j phi(K_j) over the N tokens of k, v."""
    torch = _torch()
    _dev(k, "k")
    _dev(v, "v")
    B, H, N, D = k.shape
    M = v.shape[3]
    dt = _dtype_code(k)
    if S is None:
        S = torch.empty((B, H, D, M), dtype=torch.float32, device=k.device)
    if Z is None:
        Z = torch.empty((B, H, D), dtype=torch.float32, device=k.device)
    lib = _native.load()
    need = int(lib.la_workspace_bytes(_native.LA_OP_PREFIX_STATE, B, H, N, D, M, 1, dt))
    ws = _workspace(need, k.device)
    wsz = 0 if ws is None else ws.numel()
    _native.check(lib.la_prefix_state(k.data_ptr(), v.data_ptr(), S.data_ptr(), Z.data_ptr(), B, H, N, D, M, dt,
                                      _ptr(ws), wsz, _stream(stream)))
    return S, Z
