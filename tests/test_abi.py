"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol include/linattn.h declares, and rejects bad arguments before any HIP
call.  Pointers below are fake addresses; every call is built so that
validation fails first, and the tests are skipped on a host with a GPU."""

import ctypes
import os
import re

import pytest

from kernelized_causal_attention_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")


def _gpu_visible() -> bool:
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_native.LIB_PATH):
        from kernelized_causal_attention_amd import build

        build.build(verbose=False)
    return _native.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_symbols()
    for required in ("la_forward", "la_backward", "la_decode_step"):
        assert required in names
    assert set(names) == set(_native.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.la_status_str(0) == b"LA_OK"
    assert lib.la_status_str(1) == b"LA_ERR_INVALID"
    assert lib.la_status_str(2) == b"LA_ERR_UNSUPPORTED"
    assert lib.la_status_str(3) == b"LA_ERR_DEVICE"
    assert lib.la_version() >= 100


def test_workspace_bytes(lib):
    # causal forward over one segment needs nothing; non-causal needs the
    # per-segment records and a total; backward always needs records + den.
    one = _native.la_plan(0, 1, 1)
    assert lib.la_workspace_bytes_ex(0, 1, 1, 64, 16, 16, 1, 0, ctypes.byref(one)) == 0
    nc = lib.la_workspace_bytes_ex(0, 1, 1, 64, 16, 16, 0, 0, ctypes.byref(one))
    assert nc >= 2 * (16 * 16 + 16) * 4
    bw = lib.la_workspace_bytes(1, 2, 3, 100, 8, 4, 1, 0)
    assert bw >= 2 * 3 * 100 * 4
    assert lib.la_workspace_bytes(3, 2, 3, 1, 8, 4, 1, 0) == 0  # decode
    assert lib.la_workspace_bytes(0, 1, 1, 64, 300, 16, 1, 0) == 0  # unsupported -> 0


def test_resolve_plan(lib):
    out = _native.la_plan()
    st = lib.la_resolve_plan(0, 4, 8, 2048, 64, 64, 1, 0, None, ctypes.byref(out))
    assert st == 0
    assert out.segments >= 1 and out.chunk in (16, 32, 64) and out.kernel in (1, 2)
    req = _native.la_plan(16, 3, 1)
    assert lib.la_resolve_plan(0, 1, 1, 1000, 16, 16, 1, 0, ctypes.byref(req), ctypes.byref(out)) == 0
    assert (out.chunk, out.segments, out.kernel) == (16, 3, 1)
    bad = _native.la_plan(48, 0, 1)
    assert lib.la_resolve_plan(0, 1, 1, 100, 16, 16, 1, 0, ctypes.byref(bad), ctypes.byref(out)) == 1
    bad = _native.la_plan(0, 0, 7)
    assert lib.la_resolve_plan(0, 1, 1, 100, 16, 16, 1, 0, ctypes.byref(bad), ctypes.byref(out)) == 1
    # bf16 D = M = 128: MFMA kernels up to 2^31 bytes per head, generic beyond
    assert lib.la_resolve_plan(0, 1, 1, (1 << 23) - 64, 128, 128, 1, 1, None, ctypes.byref(out)) == 0
    assert out.kernel == 2
    assert lib.la_resolve_plan(0, 1, 1, 1 << 23, 128, 128, 1, 1, None, ctypes.byref(out)) == 0
    assert out.kernel == 1
    mf = _native.la_plan(0, 0, 2)
    assert lib.la_resolve_plan(0, 1, 1, 1 << 23, 128, 128, 1, 1, ctypes.byref(mf), ctypes.byref(out)) == 2


def test_backward_plan_cuts_segments_like_the_forward(lib):
    # The forward's saved records are per segment of its plan, so the
    # backward of the same call must cut the sequence the same way, also where
    # the two ops run different kernel families: fp32 at D = M = 64 has an
    # MFMA forward but only the generic backward.  Checked through the
    # resolved segment counts and the saved-state size the forward reports.
    fwd, bwd = _native.la_plan(), _native.la_plan()
    for dtype, D in ((0, 64), (0, 32), (0, 128), (1, 64), (1, 128), (1, 48)):
        for causal in (1, 0):
            for N in (1104, 1435, 2048, 700, 64, 33):
                for segs in (0, 1, 3, 5):
                    req = _native.la_plan(0, segs, 0)
                    assert lib.la_resolve_plan(0, 2, 2, N, D, D, causal, dtype, ctypes.byref(req), ctypes.byref(fwd)) == 0
                    assert lib.la_resolve_plan(1, 2, 2, N, D, D, causal, dtype, ctypes.byref(req), ctypes.byref(bwd)) == 0
                    assert fwd.segments == bwd.segments, (dtype, D, causal, N, segs, fwd.segments, bwd.segments)
    # fp32 D = 64: MFMA forward, generic backward, on the forward's segments
    req = _native.la_plan(0, 5, 0)
    assert lib.la_resolve_plan(0, 2, 2, 1104, 64, 64, 1, 0, ctypes.byref(req), ctypes.byref(fwd)) == 0
    assert lib.la_resolve_plan(1, 2, 2, 1104, 64, 64, 1, 0, ctypes.byref(req), ctypes.byref(bwd)) == 0
    assert (fwd.kernel, bwd.kernel, fwd.segments, bwd.segments) == (2, 1, 5, 5)


def test_resolve_plan_chunk_128(lib):
    # 128-token chunks: the bf16 MFMA forward at D = M = 64 only; segments are
    # whole 128-token chunks (for every op of a call with that plan, so the
    # backward cuts the sequence as the forward did)
    out = _native.la_plan()
    for op in (0, 1):
        for N in (1000, 8192, 300, 129):
            for segs in (0, 3, 6):
                req = _native.la_plan(128, segs, 0)
                assert lib.la_resolve_plan(op, 2, 4, N, 64, 64, 1, 1, ctypes.byref(req), ctypes.byref(out)) == 0
                assert out.chunk == 128 and out.kernel == 2
                assert out.segments <= -(-N // 128)
    req = _native.la_plan(128, 6, 0)
    base = _native.la_plan(64, 6, 0)
    o128, o64 = _native.la_plan(), _native.la_plan()
    assert lib.la_resolve_plan(0, 1, 1, 1000, 64, 64, 1, 1, ctypes.byref(req), ctypes.byref(o128)) == 0
    assert lib.la_resolve_plan(0, 1, 1, 1000, 64, 64, 1, 1, ctypes.byref(base), ctypes.byref(o64)) == 0
    # 1000 tokens in six pieces: 192-token segments (6) in 64-token units, 256 (4) in 128-token units
    assert (o64.segments, o128.segments) == (6, 4)
    for bad_args in ((0, 1, 1, 1000, 128, 128, 1, 1), (0, 1, 1, 1000, 64, 64, 1, 0),
                     (0, 1, 1, 1000, 32, 32, 1, 1)):
        assert lib.la_resolve_plan(*bad_args, ctypes.byref(req), ctypes.byref(out)) == 1
    gen = _native.la_plan(128, 0, 1)
    assert lib.la_resolve_plan(0, 1, 1, 1000, 64, 64, 1, 1, ctypes.byref(gen), ctypes.byref(out)) == 1


def test_poly_workspace_and_support(lib):
    # the polynomial backward keeps one float per row (c_i); other dtypes or
    # sizes are unsupported (0 bytes)
    assert lib.la_workspace_bytes(_native.LA_OP_POLY_BACKWARD, 2, 3, 100, 64, 64, 1, 1) >= 2 * 3 * 100 * 4
    assert lib.la_workspace_bytes(_native.LA_OP_POLY_BACKWARD, 2, 3, 100, 64, 64, 1, 0) == 0
    assert lib.la_workspace_bytes(_native.LA_OP_POLY_BACKWARD, 2, 3, 100, 32, 32, 1, 1) == 0


def test_retention_plan_and_anchor_workspace(lib):
    # the retention calls take the linear-attention plan (512 heads fill the
    # chip with one segment each); the backward anchors its gate gradients
    # every 1024 tokens inside a segment as well, keeping one fp32 D x M
    # state and one scalar per inner anchor in its workspace
    out = _native.la_plan()
    for op in (_native.LA_OP_RETENTION_FORWARD, _native.LA_OP_RETENTION_BACKWARD, _native.LA_OP_FORWARD):
        assert lib.la_resolve_plan(op, 4, 128, 8192, 64, 64, 1, 1, None, ctypes.byref(out)) == 0
        assert out.segments == 1 and out.kernel == 2
        assert lib.la_resolve_plan(op, 8, 16, 8192, 64, 64, 1, 1, None, ctypes.byref(out)) == 0
        assert out.segments == 4
    # the saved record: one state (D*M + D floats) per segment
    assert lib.la_retention_saved_bytes(4, 128, 8192, 64, 64, 1) == 512 * 1 * (64 * 64 + 64) * 4
    assert lib.la_retention_saved_bytes(8, 16, 8192, 64, 64, 1) == 128 * 4 * (64 * 64 + 64) * 4
    assert lib.la_retention_saved_bytes(4, 128, 8192, 64, 64, 0) == 0  # fp32: no retention kernels
    # backward workspace (regions of 256-byte multiples): segment and suffix
    # records, the per-token a, and at 8192 tokens per segment 7 inner anchors
    rec = 512 * 1 * (64 * 64 + 64) * 4
    want = 2 * rec + 512 * 8192 * 4 + 512 * 7 * 64 * 64 * 4 + 512 * 7 * 4
    assert lib.la_workspace_bytes(_native.LA_OP_RETENTION_BACKWARD, 4, 128, 8192, 64, 64, 1, 1) == want
    # 1024-token segments have no inner anchor
    want = 2 * rec + 512 * 1024 * 4
    assert lib.la_workspace_bytes(_native.LA_OP_RETENTION_BACKWARD, 4, 128, 1024, 64, 64, 1, 1) == want


nogpu = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation tests run on hosts without a GPU")

A = 0x10000000  # fake, 256-byte aligned "device" addresses, far apart
Bp = 0x20000000
C = 0x30000000
Dp = 0x40000000


@nogpu
def test_forward_rejects_bad_arguments(lib):
    def fwd(q=A, k=Bp, v=C, out=Dp, B=1, H=1, N=8, D=4, M=4, causal=1, dtype=0, den=None, ws=None, wsz=0):
        return lib.la_forward(q, k, v, out, B, H, N, D, M, causal, dtype, den, ws, wsz, None)

    assert fwd(q=None) == 1 and b"q is NULL" in lib.la_last_error()
    assert fwd(out=None) == 1
    assert fwd(N=0) == 1 and b"sizes" in lib.la_last_error()
    assert fwd(B=-1) == 1
    assert fwd(dtype=5) == 1 and b"dtype" in lib.la_last_error()
    assert fwd(D=300) == 2 and b"D=300" in lib.la_last_error()
    assert fwd(D=200, M=200) == 2
    assert fwd(q=A + 2) == 1 and b"aligned" in lib.la_last_error()  # fp32 needs 4-byte alignment
    assert fwd(out=A + 64) == 1 and b"overlaps" in lib.la_last_error()
    assert fwd(den=A) == 1 and b"overlaps" in lib.la_last_error()
    # non-causal always needs a workspace: none given -> rejected before launch
    assert fwd(causal=0) == 1 and b"workspace" in lib.la_last_error()
    need = lib.la_workspace_bytes(0, 1, 1, 8, 4, 4, 0, 0)
    assert fwd(causal=0, ws=0x50000000, wsz=need - 1) == 1 and b"too small" in lib.la_last_error()


@nogpu
def test_backward_rejects_bad_arguments(lib):
    E = 0x50000000
    F = 0x60000000
    G = 0x70000000
    H_ = 0x80000000

    def bwd(dq=F, dk=G, dv=H_, ws=None, wsz=0, N=8, den=None):
        return lib.la_backward(A, Bp, C, Dp, E, den, dq, dk, dv, 1, 1, N, 4, 4, 1, 0, ws, wsz, None)

    assert bwd(dq=None) == 1
    assert bwd(dk=A) == 1 and b"overlaps" in lib.la_last_error()
    assert bwd(dv=F) == 1 and b"overlap" in lib.la_last_error()
    assert bwd() == 1 and b"workspace" in lib.la_last_error()  # backward needs a workspace
    need = lib.la_workspace_bytes(1, 1, 1, 8, 4, 4, 1, 0)
    assert bwd(ws=0x90000000, wsz=need - 4) == 1 and b"too small" in lib.la_last_error()


@nogpu
def test_decode_and_prefix_reject_bad_arguments(lib):
    assert lib.la_decode_step(None, Bp, C, Dp, A + 0x100000, 0x50000000, 2, 2, 4, 4, 0, None) == 1
    # out overlapping q
    assert lib.la_decode_step(A, Bp, C, Dp, 0x50000000, C + 4, 2, 2, 4, 4, 0, None) == 1
    assert b"overlaps" in lib.la_last_error()
    assert lib.la_decode_step(A, Bp, C, Dp, 0x50000000, 0x60000000, 2, 2, 4, 512, 0, None) == 2
    assert lib.la_prefix_state(A, Bp, None, Dp, 1, 1, 8, 4, 4, 0, None, 0, None) == 1
    assert lib.la_prefix_state(A, Bp, A, Dp, 1, 1, 8, 4, 4, 0, None, 0, None) == 1


def test_binding_requires_built_library_loudly(monkeypatch, tmp_path):
    # With the library path pointing nowhere, loading raises instead of
    # falling back to anything.
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _native.load()


def test_saved_bytes(lib):
    # causal over one segment keeps nothing; several segments keep one record
    # (S, Z: D*M + D floats) per segment and head; non-causal keeps the totals.
    one = _native.la_plan(0, 1, 1)
    four = _native.la_plan(0, 4, 1)
    E = 16 * 8 + 16
    assert lib.la_saved_bytes(1, 1, 256, 16, 8, 1, 0, ctypes.byref(one)) == 0
    assert lib.la_saved_bytes(2, 3, 256, 16, 8, 1, 0, ctypes.byref(four)) == 2 * 3 * 4 * E * 4
    assert lib.la_saved_bytes(2, 3, 256, 16, 8, 0, 0, ctypes.byref(four)) == 2 * 3 * E * 4
    assert lib.la_saved_bytes(1, 1, 256, 300, 8, 1, 0, None) == 0  # unsupported -> 0


@nogpu
def test_saved_state_arguments_are_validated(lib):
    E = 0x50000000
    F = 0x60000000
    G = 0x70000000
    H_ = 0x80000000
    S = 0xA0000000
    W = 0xB0000000
    four = _native.la_plan(0, 4, 1)
    need = lib.la_saved_bytes(1, 1, 256, 4, 4, 1, 0, ctypes.byref(four))
    fws = lib.la_workspace_bytes_ex(0, 1, 1, 256, 4, 4, 1, 0, ctypes.byref(four))

    def fwd(saved=S, ssz=need, plan=four):
        return lib.la_forward_ex(A, Bp, C, Dp, 1, 1, 256, 4, 4, 1, 0, None, saved, ssz, W, fws, None,
                                 ctypes.byref(plan))

    assert fwd(saved=S + 4) == 1 and b"16-byte" in lib.la_last_error()
    assert fwd(ssz=need - 4) == 1 and b"saved too small" in lib.la_last_error()
    assert fwd(saved=C) == 1 and b"saved overlaps input v" in lib.la_last_error()

    bws = lib.la_workspace_bytes_ex(1, 1, 1, 256, 4, 4, 1, 0, ctypes.byref(four))

    def bwd(saved=S, ssz=need, plan=four, dq=F):
        return lib.la_backward_ex(A, Bp, C, Dp, E, None, saved, ssz, dq, G, H_, 1, 1, 256, 4, 4, 1, 0, W, bws,
                                  None, ctypes.byref(plan))

    assert bwd(ssz=need - 4) == 1 and b"saved too small" in lib.la_last_error()
    assert bwd(dq=S) == 1 and b"overlaps input saved" in lib.la_last_error()


@nogpu
def test_fp32_backward_takes_the_forwards_saved_states(lib):
    # fp32 D = M = 64 on the automatic plan: the MFMA forward keeps its
    # segment states, and the generic backward must accept them (the same
    # segments).  The call is given a workspace that is too small, so it stops
    # after the saved-state checks, before any HIP call: the error it reports
    # is the workspace's, not a segment mismatch.
    A, Bp, C, Dp, E, F, G, H_, S, W = (0x10000000 * (n + 1) for n in range(10))
    for N, causal, segs in ((1104, 1, 5), (1435, 0, 0), (2048, 1, 0), (700, 1, 3)):
        plan = _native.la_plan(0, segs, 0)
        ssz = lib.la_saved_bytes(2, 2, N, 64, 64, causal, 0, ctypes.byref(plan))
        assert ssz > 0
        st = lib.la_backward_ex(A, Bp, C, Dp, E, None, S, ssz, F, G, H_, 2, 2, N, 64, 64, causal, 0, W, 1, None,
                                ctypes.byref(plan))
        assert st == 1 and b"workspace too small" in lib.la_last_error(), (N, causal, segs, lib.la_last_error())


@nogpu
def test_misaligned_tensors_leave_the_mfma_kernels(lib):
    # The MFMA kernels move q, k, v, out, dout, dq, dk, dv in 16-byte vectors.
    # A bf16 pointer that is only 2-byte aligned is valid, but on the
    # automatic plan it must run the generic kernels (cut into the same
    # segments), and a plan that forces the MFMA kernels is refused.  The
    # routing shows in the workspace a backward asks for: the MFMA sweeps also
    # pass c_i between them (one float per row) and keep hand-off flags, the
    # generic ones do not.
    E = 0x50000000
    F = 0x60000000
    G = 0x70000000
    H_ = 0x80000000
    W = 0xB0000000
    N = 256
    mf = lib.la_workspace_bytes(1, 1, 1, N, 64, 64, 1, 1)  # sizes assume aligned pointers: MFMA
    out = _native.la_plan()
    assert lib.la_resolve_plan(1, 1, 1, N, 64, 64, 1, 1, None, ctypes.byref(out)) == 0 and out.kernel == 2
    generic = _native.la_plan(0, out.segments, 1)
    generic_need = lib.la_workspace_bytes_ex(1, 1, 1, N, 64, 64, 1, 1, ctypes.byref(generic))
    assert generic_need < mf

    def bwd(q=A, dv=H_, plan=None):
        return lib.la_backward_ex(q, Bp, C, Dp, E, None, None, 0, F, G, dv, 1, 1, N, 64, 64, 1, 1, W, 64,
                                  None, None if plan is None else ctypes.byref(plan))

    assert bwd() == 1 and f"{mf} needed".encode() in lib.la_last_error()
    assert bwd(q=A + 2) == 1 and f"{generic_need} needed".encode() in lib.la_last_error()
    assert bwd(dv=H_ + 8) == 1 and f"{generic_need} needed".encode() in lib.la_last_error()
    # the workspace the sizing query reports covers the routed call too
    assert generic_need <= mf
    forced = _native.la_plan(0, 0, 2)
    assert bwd(q=A + 2, plan=forced) == 2 and b"16-byte" in lib.la_last_error()

    def fwd(q=A, out=Dp, plan=None):
        return lib.la_forward_ex(q, Bp, C, out, 1, 1, N, 64, 64, 1, 1, None, None, 0, None, 0, None,
                                 None if plan is None else ctypes.byref(plan))

    assert fwd(out=Dp + 2, plan=forced) == 2 and b"16-byte" in lib.la_last_error()
    # odd addresses stay invalid for bf16 (element alignment)
    assert fwd(q=A + 1) == 1 and b"aligned" in lib.la_last_error()


@nogpu
def test_families_without_generic_kernels_need_16_byte_alignment(lib):
    E = 0x50000000
    F = 0x60000000
    G = 0x70000000
    H_ = 0x80000000
    L = 0x90000000
    N = 256
    assert lib.la_poly_forward(A + 2, Bp, C, Dp, None, 1, 1, N, 64, 64, 1, 1, None) == 2
    assert b"16-byte" in lib.la_last_error()
    assert lib.la_softmax_forward(A, Bp, C, Dp + 2, None, 1, 1, N, 64, 64, 1, 1, None) == 2
    assert b"16-byte" in lib.la_last_error()
    assert lib.la_retention_forward(A, Bp + 2, C, L, Dp, 1, 1, N, 64, 64, 1, None, None, None, 0, None, 0,
                                    None) == 2
    assert b"16-byte" in lib.la_last_error()
    assert lib.la_poly_backward(A, Bp, C, Dp, E, L, F + 2, G, H_, 1, 1, N, 64, 64, 1, 1, 0xB0000000, 1 << 20,
                                None) == 2
    assert b"16-byte" in lib.la_last_error()


@nogpu
def test_noalloc_forward_rejects_calls_beyond_its_scratch(lib):
    # la_forward_noalloc keeps its segment records in a 64 MiB static device
    # array; a call that needs more is refused before any HIP call
    B, H, N, D = 4, 256, 64, 128
    assert lib.la_workspace_bytes(0, B, H, N, D, D, 0, 1) > 64 << 20
    st = lib.la_forward_noalloc(A, Bp, C, Dp, B, H, N, D, D, 0, 1, None, None)
    assert st == 2 and b"static scratch" in lib.la_last_error()
    assert lib.la_forward_noalloc(None, Bp, C, Dp, 1, 1, 8, 4, 4, 1, 0, None, None) == 1
