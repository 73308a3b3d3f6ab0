"""Benchmark: causal linear attention forward+backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

A step is one pass of the training hot path over one batch: la_forward
(causal, keeping the row denominators and the per-segment prefix states)
followed by la_backward reading those states, on the
bf16 workload B=8, H=16, N=8192, D=M=64 (Q, K, V ~ N(0,1)/sqrt(D), dout ~
N(0,1), synthetic, drawn on the device, resident in HBM before timing).
The timed region is exactly K steps between two synchronisations, timed with
HIP events on the working stream.  Prints ONE JSON line.

Extra fields:
  roofline      -- the step's algorithmic HBM bytes (inputs read once, outputs
                   written once, per head-token: 512 forward + 1024 backward
                   + 8 for the saved denominator at D = M = 64 in bf16) over
                   the measured step time, against 8 TB/s; `traffic` is the
                   step's HBM bytes from the committed rocprofv3 FETCH_SIZE /
                   WRITE_SIZE table (null when it was taken on other kernel
                   sources); `mfma` gives TFLOP/s under the algorithmic,
                   useful-executed and executed flop counts and the counted
                   MFMA flops and busy fraction per kernel; `dominant_kernel`
                   is the longest kernel's own I/O over its HIP-event time.
  kernels       -- every kernel of the step: launches, time, own I/O, GB/s.
  long_bf16     -- the long-sequence forward (B=1, H=16, N=65536, D=M=128).
  fwd_f32       -- the fp32 forward (B=4, H=8, N=2048, D=M=64), warm and with
                   the caches scrubbed between calls.
  cpu_baseline  -- the fp64 oracle (test infrastructure, timed here only) on
                   the host's cores, before any GPU work: a pool of
                   single-threaded processes, one head per task, on the
                   headline workload (all 128 heads), the long-sequence
                   forward (all 16 heads) and 8 decode steps (all heads).
  decode        -- the batched decode step (B=256, H=32, D=M=128, fp32 state,
                   1024 consecutive steps after a 512-token prefix): steps/s
                   and HBM GB/s.
  retention     -- decayed / gated linear attention forward+backward on the
                   same shape (gates gamma_t ~ U(0.6, 1)): tokens/s and the
                   dominant kernel's HBM roofline.
  poly          -- degree-2 polynomial-kernel attention forward+backward on
                   the same shape: tokens/s and the dominant kernel's MFMA
                   roofline (TFLOP/s against the dense bf16 peak).
  softmax       -- the softmax baseline's causal forward on the same shape,
                   beside the linear-attention forward on the same inputs;
                   the decode field adds the softmax KV-cache step on the
                   decode workload's tokens and the linear decode's speedup.
"""

from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3  # MI355X fp32 matrix / vector, published


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the decode measurement")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--retention-only", action="store_true",
                    help="run only the retention forward+backward measurement (for profiling) and print it")
    ap.add_argument("--poly-only", action="store_true",
                    help="run only the polynomial-kernel forward+backward measurement (for profiling) and print it")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps (the GPU raises its clocks "
                         "over the first few hundred milliseconds of load)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration under rocprofv3)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only run the streaming-bandwidth microbenchmark and print its lines")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-bandwidth microbenchmark (e.g. under a profiler)")
    ap.add_argument("--only", choices=["fwdbwd_bf16", "long_bf16", "fwd_f32", "decode_f32", "chunk128"],
                    help="run only this workload's measurement (for profiling) and print it")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle baseline worker processes (0: the cores this process may run on, at most 16)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                    help="summarise rocprofv3 --pmc counter_collection CSV files (per kernel, per dispatch) "
                         "into a table, then exit")
    ap.add_argument("--pmc-calib", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="with --pmc-summary: FETCH_SIZE / WRITE_SIZE of --calibrate-copy, to scale those "
                         "counters to bytes")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarise a rocprofv3 --kernel-trace kernel_trace CSV: per library kernel and grid "
                         "size, calls, average / min / max duration and the kernel's registers and LDS, then exit")
    ap.add_argument("--pmc-out", help="with --pmc-summary: write the table here (default: stdout)")
    ap.add_argument("--pmc-title", default="", help="with --pmc-summary: the table's first comment line")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="with --pmc-summary: a command line recorded in the table's header (repeatable)")
    return ap.parse_args()


CEILING_EXE = os.path.join(ROOT, "kernelized_causal_attention_amd", "_lib", "hbm_ceiling")
# the traffic mix of each kernel (tensors read / written), for its practical ceiling
KERNEL_MIX = {"mfma.seg_state": "r2", "mfma.forward": "r3w1", "mfma.forward_t128": "r3w1", "mfma.bwd_dq": "r4w1",
              "mfma.bwd_dkdv": "r4w2", "decode": "r1w1"}


def hbm_ceilings():
    """Streaming rates of plain 16-byte-vector kernels for each traffic mix,
    measured on this GPU by a child process (the parent has not touched the
    GPU yet).  Returns {mix: GB/s}, or None when the program is missing."""
    if not os.path.exists(CEILING_EXE):
        log(f"{CEILING_EXE} missing (build first): no practical ceilings")
        return None
    try:
        r = subprocess.run([CEILING_EXE], capture_output=True, text=True, timeout=120)
    except (OSError, subprocess.TimeoutExpired) as e:
        log(f"hbm_ceiling did not run: {e}")
        return None
    if r.returncode != 0:
        log(f"hbm_ceiling failed ({r.returncode}): {r.stderr.strip()[-300:]}")
        return None
    mixes = {}
    for line in r.stdout.splitlines():
        d = json.loads(line)
        if "mix" in d:
            mixes[d["mix"]] = d["GBps"]
        elif "mfma" in d:
            MFMA_CEIL[d["mfma"]] = d["TFLOPs"]
    log("streaming ceilings (GB/s): " + ", ".join(f"{k} {v:.0f}" for k, v in mixes.items()))
    if MFMA_CEIL:
        log("matrix-core ceilings (TFLOP/s): " + ", ".join(f"{k} {v:.0f}" for k, v in MFMA_CEIL.items()))
    return mixes


# measured register-only MFMA loop rates, filled by hbm_ceilings()
MFMA_CEIL = {}


def with_mfma_ceiling(roof, key="bf16_16x16x32"):
    """Adds the measured matrix-core ceiling to an MFMA-bound roofline."""
    c = MFMA_CEIL.get(key)
    if c:
        roof["measured_ceiling"] = c
        roof["frac_of_measured_ceiling"] = round(roof["achieved"] / c, 4)
    return roof


# ---------------------------------------------------------------- bytes ----
def kernel_bytes(name: str, B, H, N, D, M, es, P=1):
    """Algorithmic HBM bytes one launch of `name` must move (inputs read once,
    outputs written once), for B*H heads of N tokens."""
    ht = B * H * N
    # the causal forward's segment-state pass reads the first P - 1 segments
    # (the last one's aggregate would only feed the total), and its scan reads
    # P - 1 records and writes P
    ht_agg = ht * (P - 1) // P if P > 1 else ht
    seg_len = -(-(-(-N // 64)) // P) * 64
    anchors = B * H * P * ((seg_len - 1) // 1024)  # retention backward's inner anchors
    family, _, base = name.rpartition(".")
    if family == "ret":
        # decayed / gated linear attention; the log gammas are 4 bytes a token
        if base == "seg_state":
            return ht_agg * (es * (D + M) + 4)
        if base == "scan":
            return B * H * (P * 2 - 1) * D * M * 4
        if base == "rscan":
            return B * H * (P * 2 + 1) * D * M * 4
        if base == "forward":
            return ht * (es * (2 * D + M) + 4 + es * M)
        if base == "bwd_dq":  # reads q, k, v, dy, gates; writes dq, a and the anchor states
            return ht * (es * (2 * D + 2 * M) + 4 + es * D + 4) + anchors * D * M * 4
        if base == "bwd_dkdv":  # reads q, k, v, dy, gates, a and the anchor states; writes dk, dv, a
            return ht * (es * (2 * D + 2 * M) + 4 + 8 + es * (D + M)) + anchors * D * M * 4
        if base == "dlg":  # reads a and the segment-end states S, R; writes d log gamma
            return ht * 8 + B * H * (P - 1) * 2 * D * M * 4
    if family == "mfma" and base == "bwd_dq":
        # reads q, k, v, dout; writes dq and the per-row (c, den) pair
        return ht * (es * (2 * D + 2 * M) + es * D + 8)
    if family == "mfma" and base == "bwd_fused":
        # reads q, k, v, dout once (the reverse sweep's re-reads are the same
        # tensors); writes dq, dk, dv; writes and reads back (c, den)
        return ht * (es * (2 * D + 2 * M) + es * (2 * D + M) + 16)
    if family == "mfma" and base == "bwd_dkdv":
        # reads q, k, v, dout and (c, den); writes dk, dv
        return ht * (es * (2 * D + 2 * M) + 8 + es * (D + M))
    if base in ("forward", "forward_t128"):
        return ht * (es * (2 * D + M) + es * M + 4)
    if base == "forward_den":
        return ht * (es * (2 * D + M) + 4)
    if base == "seg_state":
        return ht_agg * es * (D + M)
    if base == "bwd_dq":
        return ht * (es * (2 * D + 3 * M) + 4 + es * D)
    if base == "bwd_dkdv":
        return ht * (es * (2 * D + 3 * M) + 4 + es * (D + M))
    if base == "seg_scan":
        return B * H * (P * 2 - 1) * (D * M + D) * 4
    if base == "decode":
        return B * H * (2 * D * M * 4 + 2 * D * 4 + es * (2 * D + M) + es * M)
    return 0


def kernel_flops(name: str, B, H, N, D, M, causal=True):
    """Matrix-product flops one launch of a polynomial-kernel pass performs
    over the query-key pairs it must visit (N (N + 1) / 2 per head causal):
    forward s = q.k and P V (2D + 2M per pair); dq sweep s, g.v and dS K
    (4D + 2M); dk / dv sweep s, g.v, P^T g and dS^T q (4D + 4M)."""
    pairs = B * H * (N * (N + 1) // 2 if causal else N * N)
    per = {"poly.forward": 2 * D + 2 * M, "poly.bwd_dq": 4 * D + 2 * M, "poly.bwd_dkdv": 4 * D + 4 * M}
    return pairs * per.get(name, 0)


# ------------------------------------------------- algorithmic counts ----
# Per head-token (ht), the path's own inputs read once and outputs written
# once, at the stored widths: the forward reads q, k, v and writes out; the
# backward reads q, k, v, out, dout and writes dq, dk, dv; a training step
# also writes the fp32 row denominator in the forward and reads it in the
# backward (8 bytes).
def alg_bytes_per_ht(kind, D, M, es):
    fwd = es * (2 * D + M) + es * M
    if kind == "fwd":
        return fwd
    if kind == "fwdbwd":
        return fwd + es * (2 * D + 3 * M) + es * (2 * D + M) + 8
    raise ValueError(kind)


def flops_per_ht(kind, D, M, T=64):
    """Flops per head-token under three counts: algorithmic (the method's
    two O(N C M) products forward, 4 D M; the backward's five, 10 D M),
    useful-executed (plus the causal half of the intra-chunk T x T tiles) and
    executed (full T x T tiles)."""
    alg = {"fwd": 4 * D * M, "fwdbwd": 14 * D * M}[kind]
    # intra-chunk products per row: forward scores and A.V (2 T (D + M)),
    # backward six of them (6 T (D + M)); the causal half keeps (T + 1) / 2 keys
    intra = {"fwd": 2 * (D + M), "fwdbwd": 8 * (D + M)}[kind]
    return {"algorithmic": alg, "useful_executed": alg + intra * (T + 1) / 2, "executed": alg + intra * T}


def timed_steps(la, torch, step, steps, warmup, settle=0.0, nbreak=3):
    """Settle, warm up, time every kernel over `nbreak` steps (breakdown),
    then time exactly `steps` steps between two synchronisations with HIP
    events on the working stream, bracketing only the dominant kernel.
    Returns (ms per step, breakdown {name: (launches, ms)}, dominant name,
    dominant average ms)."""
    t_settle = time.time() + settle
    while time.time() < t_settle:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    la.profile_enable(True)
    for _ in range(nbreak):
        step()
    torch.cuda.synchronize()
    prof = la.profile_report()
    kname = max(prof.items(), key=lambda kv: kv[1][1])[0]
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    la.profile_enable(True, only=kname)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    nl, tot_ms = la.profile_report()[kname]
    la.profile_enable(False)
    return t0.elapsed_time(t1) / steps, prof, kname, tot_ms / nl


def per_iteration_ms(torch, fn, n, warmup=3):
    """Median and min over n iterations, each bracketed by HIP events on
    the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2]), t[0]


def kernel_table(prof, nbreak, B, H, N, D, M, es, P, ceil=None):
    """Per-kernel breakdown: launches per step, average time and the
    kernel's own HBM I/O (inputs it reads once, outputs it writes once)."""
    kernels = {}
    for name, (n, t) in sorted(prof.items()):
        b = kernel_bytes(name, B, H, N, D, M, es, P)
        avg = t / n
        kernels[name] = {"launches_per_step": n / nbreak, "avg_ms": round(avg, 4),
                         "own_io_bytes": b, "GBps": round(b / (avg / 1e3) / 1e9, 1) if b else None}
        mix = KERNEL_MIX.get(name)
        if ceil and mix in ceil and b:
            kernels[name]["ceiling_mix"] = mix
            kernels[name]["frac_of_ceiling"] = round(b / (avg / 1e3) / 1e9 / ceil[mix], 4)
    return kernels


def step_roofline(kind, B, H, N, D, M, es, ms, kernels, traffic_file, counters_file, what):
    """The section 8(d) roofline of one step: algorithmic bytes per step over
    the measured step time, against 8 TB/s; HBM traffic per step from the
    committed counter table (launches per step x bytes per launch); the MFMA
    view under the three flop counts, with the hardware-counted MFMA flops
    and busy fraction per kernel when the committed counter table matches
    these kernel sources."""
    ht = B * H * N
    alg = alg_bytes_per_ht(kind, D, M, es) * ht
    achieved = alg / (ms / 1e3) / 1e9
    traffic = None
    tt = read_profile_table(traffic_file)
    if tt is not None and all(name in tt for name in kernels):
        traffic = int(sum(k["launches_per_step"] * (tt[name][0] + tt[name][1]) for name, k in kernels.items()))
    fl = flops_per_ht(kind, D, M)
    tfl = {c: round(f * ht / (ms / 1e3) / 1e12, 1) for c, f in fl.items()}
    ai = fl["algorithmic"] / alg_bytes_per_ht(kind, D, M, es)
    mfma = {"unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS if es == 2 else PEAK_F32_TFLOPS,
            "achieved": tfl,
            "frac_of_peak": {c: round(v / (PEAK_BF16_TFLOPS if es == 2 else PEAK_F32_TFLOPS), 4)
                             for c, v in tfl.items()},
            "algorithmic_intensity_flop_per_byte": round(ai, 1),
            "attainable_at_hbm_peak_TFLOPs": round(min(PEAK_BF16_TFLOPS if es == 2 else PEAK_F32_TFLOPS,
                                                       ai * PEAK_HBM_GBS / 1e3), 1),
            "note": "every pass is HBM-bound at this shape (intensity far below the ridge point), so the "
                    "binding roofline is HBM bandwidth"}
    mc = MFMA_CEIL.get("bf16_16x16x32" if es == 2 else "f32_16x16x4")
    if mc:
        mfma["measured_ceiling"] = mc
        mfma["frac_of_measured_ceiling"] = {c: round(v / mc, 4) for c, v in tfl.items()}
    ct = read_profile_table(counters_file, cols=None)
    if ct is not None:
        per = {}
        step_flops = 0.0
        for name, k in kernels.items():
            row = ct.get(name)
            if row is None:
                continue
            per[name] = row
            for c in ("MfmaFlopsBF16", "MfmaFlopsF32"):
                step_flops += k["launches_per_step"] * row.get(c, 0.0)
        if per:
            mfma["counters_per_kernel"] = per
            if step_flops:
                mfma["measured_TFLOPs"] = round(step_flops / (ms / 1e3) / 1e12, 1)
    return {"bound": "hbm", "kernel": what, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "traffic_over_alg": round(traffic / alg, 3) if traffic else None,
            "alg_bytes_per_step": alg, "alg_bytes_per_head_token": alg_bytes_per_ht(kind, D, M, es),
            "ms_per_step": round(ms, 4), "mfma": mfma}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(every (b,h) head is independent; multi-GPU sharding is described in the design notes, "
              "not run).", file=sys.stderr)
        sys.exit(2)
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return
    if args.ceilings:
        r = subprocess.run([CEILING_EXE])
        sys.exit(r.returncode)
    profiling = args.calibrate_copy or args.retention_only or args.poly_only or args.only
    # The oracle baseline runs first, in a pool of worker processes, while no
    # process of this run has touched the GPU yet.
    cpu = None
    if not (args.no_cpu or profiling):
        cpu = cpu_baseline(args.cpu_workers)
    ceil = None
    if not (args.no_ceiling or profiling):
        ceil = hbm_ceilings()

    import torch

    if args.calibrate_copy:
        calibrate_copy(torch)
        return

    import kernelized_causal_attention_amd as la

    torch.cuda.set_device(0)
    if args.retention_only:
        print(json.dumps(bench_retention(la, torch, args.steps, args.warmup)), flush=True)
        return
    if args.poly_only:
        print(json.dumps(bench_poly(la, torch, args.steps, args.warmup)), flush=True)
        return
    if args.only:
        fn = {"fwdbwd_bf16": lambda: bench_fwdbwd(la, torch, args, None),
              "long_bf16": lambda: bench_long(la, torch, args.steps, args.warmup, None),
              "fwd_f32": lambda: bench_fwd_f32(la, torch, args.steps, args.warmup, None),
              "decode_f32": lambda: bench_decode(la, torch, args.decode_steps),
              "chunk128": lambda: bench_chunk128(la, torch, args.steps, args.warmup)}[args.only]
        print(json.dumps(fn()), flush=True)
        return

    result = bench_fwdbwd(la, torch, args, ceil)
    if not args.no_extra:
        result["long_bf16"] = bench_long(la, torch, args.steps, args.warmup, ceil)
        result["fwd_f32"] = bench_fwd_f32(la, torch, args.steps, args.warmup, ceil)
        result["chunk_128"] = bench_chunk128(la, torch, args.steps, args.warmup)
        result["decode"] = bench_decode(la, torch, args.decode_steps)
        if ceil and "r1w1" in ceil:
            result["decode"]["roofline"]["frac_of_ceiling"] = round(
                result["decode"]["roofline"]["achieved"] / ceil["r1w1"], 4)
        result["retention"] = bench_retention(la, torch, args.steps, args.warmup)
        result["poly"] = bench_poly(la, torch, args.steps, args.warmup)
        result["softmax"] = bench_softmax(la, torch, args.steps, args.warmup)
    if cpu is not None:
        result["cpu_baseline"] = cpu
        if cpu.get("value"):
            result["cpu_baseline"]["gpu_over_oracle"] = round(result["value"] / cpu["value"], 1)
    print(json.dumps(result), flush=True)


def bench_fwdbwd(la, torch, args, ceil):
    """The headline step: la_forward (causal, keeping den and the prefix
    states) then la_backward reading them, bf16, B=8 H=16 N=8192 D=M=64."""
    from workloads import WORKLOADS, device_inputs

    w = WORKLOADS["fwdbwd_bf16"]
    B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
    es = 2
    dev = torch.device("cuda:0")
    q, k, v, g = device_inputs(B, H, N, D, M, "bf16", seed=0, scale=1.0 / D ** 0.5, device="cuda")
    plan_f = la.resolve_plan("forward", B, H, N, D, M, True, "bf16")
    plan_b = la.resolve_plan("backward", B, H, N, D, M, True, "bf16")
    ws_f = torch.empty(max(1, la.workspace_bytes("forward", B, H, N, D, M, True, "bf16")), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, la.workspace_bytes("backward", B, H, N, D, M, True, "bf16")), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, N, M), dtype=torch.bfloat16, device=dev)
    den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    nsaved = la.saved_bytes(B, H, N, D, M, True, "bf16")
    saved = torch.empty(nsaved, dtype=torch.uint8, device=dev) if nsaved else None

    def step():
        la.forward(q, k, v, causal=True, out=out, den=den, return_den=True, workspace=ws_f, saved=saved)
        return la.backward(q, k, v, out, g, den=den, causal=True, workspace=ws_b, saved=saved)

    log(f"workload fwdbwd_bf16 B={B} H={H} N={N} D={D} M={M}; plan fwd {plan_f} bwd {plan_b}")
    nbreak = 3
    ms, prof, kname, avg_ms = timed_steps(la, torch, step, args.steps, args.warmup, args.settle, nbreak)
    tokens = B * N
    value = tokens / (ms / 1e3)
    log(f"{ms:.3f} ms/step, {value:.4g} tokens/s; dominant {kname} {avg_ms:.4f} ms; breakdown: {prof}")
    P = plan_b["segments"]
    kernels = kernel_table(prof, nbreak, B, H, N, D, M, es, P, ceil)
    kb = kernel_bytes(kname, B, H, N, D, M, es, P)
    roof = step_roofline("fwdbwd", B, H, N, D, M, es, ms, kernels, TRAFFIC_FILE, COUNTERS_FILE,
                         "step: la_forward + la_backward (every launch of the fwd+bwd step)")
    roof["dominant_kernel"] = {"kernel": kname, "own_io_bytes_per_launch": kb, "avg_launch_ms": round(avg_ms, 4),
                               "GBps": round(kb / (avg_ms / 1e3) / 1e9, 1),
                               "note": "the kernel's own reads and writes, including re-reads of tensors "
                                       "another pass of the step also reads; timed with HIP events around "
                                       "each of its launches inside the timed region"}
    log(f"step roofline: {roof['achieved']:.0f} GB/s of section 8(d) bytes = {roof['frac']:.3f} of 8 TB/s; "
        f"counter traffic / algorithmic = {roof['traffic_over_alg']}")
    # each half alone (the forward keeps den and the prefix states; the
    # backward reads the ones the last forward left), and the step, per
    # iteration: median and min of 20
    phases = {}
    for name, fn in (("forward", lambda: la.forward(q, k, v, causal=True, out=out, den=den, return_den=True,
                                                    workspace=ws_f, saved=saved)),
                     ("backward", lambda: la.backward(q, k, v, out, g, den=den, causal=True, workspace=ws_b,
                                                      saved=saved)),
                     ("step", step)):
        med, mn = per_iteration_ms(torch, fn, 20)
        phases[name] = {"median_ms": round(med, 4), "min_ms": round(mn, 4)}
    log("per iteration (median / min ms): " + ", ".join(f"{n} {v['median_ms']} / {v['min_ms']}" for n, v in phases.items()))
    result = {
        "metric": "causal linear-attn fwd+bwd tokens/sec",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (Q,K,V ~ N(0,1)/sqrt(D), dout ~ N(0,1), device RNG seed 0)",
        "config": {"workload": "causal forward+backward, bf16 in / fp32 accumulate", "B": B, "H": H,
                   "N": N, "D": D, "M": M, "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)",
                   "plan_forward": plan_f, "plan_backward": plan_b},
        "roofline": roof,
        "kernels": kernels,
        "phases": phases,
    }
    if ceil:
        mix = KERNEL_MIX.get(kname)
        result["hbm_ceiling"] = {
            "source": "streaming microbenchmark on this GPU (kernelized_causal_attention_amd/_lib/hbm_ceiling): "
                      "plain 16-byte-vector kernels over 134 MB tensors, GB/s per traffic mix",
            "mixes": ceil, "dominant_mix": mix}
    if MFMA_CEIL:
        result["mfma_ceiling"] = {
            "source": "register-only loop of independent MFMAs over the whole chip (same program), TFLOP/s",
            "TFLOPs": dict(MFMA_CEIL), "spec": {"bf16_16x16x32": PEAK_BF16_TFLOPS, "f32_16x16x4": PEAK_F32_TFLOPS}}
    return result


def bench_chunk128(la, torch, steps, warmup):
    """Chunk length 64 against 128 on the fwd+bwd workload (B=8 H=16 N=8192
    D=M=64, bf16): the causal forward alone (keeping den and the prefix
    states) under each plan, and the whole step with the 128-token forward
    (the backward kernels take 64-token chunks over the same segments)."""
    from workloads import WORKLOADS, device_inputs

    w = WORKLOADS["fwdbwd_bf16"]
    B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
    dev = torch.device("cuda:0")
    q, k, v, g = device_inputs(B, H, N, D, M, "bf16", seed=0, scale=1.0 / D ** 0.5, device="cuda")
    out = torch.empty((B, H, N, M), dtype=torch.bfloat16, device=dev)
    den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    res = {"workload": f"causal forward (and fwd+bwd step), bf16, B={B} H={H} N={N} D=M={D}",
           "note": "two rounds, alternating the chunk lengths; forward_kernel_ms is the forward kernel's "
                   "average over the timed steps (HIP events around its launches)"}
    runs = {64: [], 128: []}
    for _ in range(2):
        for T in (64, 128):
            plan = la.resolve_plan("forward", B, H, N, D, M, True, "bf16", dict(chunk=T))
            ws_f = torch.empty(max(1, la.workspace_bytes("forward", B, H, N, D, M, True, "bf16", plan)),
                               dtype=torch.uint8, device=dev)
            ws_b = torch.empty(max(1, la.workspace_bytes("backward", B, H, N, D, M, True, "bf16", plan)),
                               dtype=torch.uint8, device=dev)
            nsaved = la.saved_bytes(B, H, N, D, M, True, "bf16", plan)
            saved = torch.empty(nsaved, dtype=torch.uint8, device=dev) if nsaved else None

            def fwd():
                la.forward(q, k, v, causal=True, out=out, den=den, return_den=True, workspace=ws_f, saved=saved,
                           plan=plan)

            def step():
                fwd()
                return la.backward(q, k, v, out, g, den=den, causal=True, workspace=ws_b, saved=saved, plan=plan)

            ms_f, prof_f, kname, avg_f = timed_steps(la, torch, fwd, steps, warmup, settle=0.5)
            ms_s, _, _, _ = timed_steps(la, torch, step, steps, warmup, settle=0.5)
            runs[T].append({"plan": plan, "forward_ms": round(ms_f, 4), "forward_kernel": kname,
                            "forward_kernel_ms": round(avg_f, 4), "step_ms": round(ms_s, 4),
                            "forward_breakdown_ms": {kk: round(tt / nn, 4) for kk, (nn, tt) in sorted(prof_f.items())}})
            log(f"chunk {T}: forward {ms_f:.4f} ms ({kname} {avg_f:.4f} ms), step {ms_s:.4f} ms")
    for T in (64, 128):
        res[f"T{T}"] = runs[T]
    return res


def bench_long(la, torch, steps, warmup, ceil):
    """The long-sequence causal forward, bf16, B=1 H=16 N=65536 D=M=128
    (segment aggregates, their scan, then the chunked forward carrying the
    128 x 128 fp32 state)."""
    from workloads import WORKLOADS, device_inputs

    w = WORKLOADS["long_bf16"]
    B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
    q, k, v, _ = device_inputs(B, H, N, D, M, "bf16", seed=0, scale=1.0 / D ** 0.5, device="cuda",
                               with_dout=False)
    out = torch.empty_like(v)
    plan = la.resolve_plan("forward", B, H, N, D, M, True, "bf16")
    ws = torch.empty(max(1, la.workspace_bytes("forward", B, H, N, D, M, True, "bf16")), dtype=torch.uint8,
                     device="cuda")

    def step():
        return la.forward(q, k, v, causal=True, out=out, workspace=ws)

    ms, prof, kname, avg_ms = timed_steps(la, torch, step, steps, warmup, settle=0.3)
    kernels = kernel_table(prof, 3, B, H, N, D, M, 2, plan["segments"], ceil)
    roof = step_roofline("fwd", B, H, N, D, M, 2, ms, kernels, TRAFFIC_FILE_LONG, COUNTERS_FILE_LONG,
                         "call: la_forward (every launch of the causal forward)")
    log(f"long_bf16: {ms:.3f} ms/call, {B * N / (ms / 1e3):.4g} tokens/s, {roof['achieved']:.0f} GB/s "
        f"({roof['frac']:.3f} of 8 TB/s); breakdown {prof}")
    return {"metric": "long-sequence causal linear-attn forward tokens/sec", "value": round(B * N / (ms / 1e3), 1),
            "unit": "tokens/s", "ms_per_call": round(ms, 4),
            "config": {"workload": "long-sequence causal forward, bf16, 128 x 128 fp32 state per head", "B": B,
                       "H": H, "N": N, "D": D, "M": M, "plan": plan},
            "roofline": roof, "kernels": kernels}


def bench_fwd_f32(la, torch, steps, warmup, ceil):
    """The fp32 causal forward, B=4 H=8 N=2048 D=M=64.  Its 64 MiB of inputs
    fit the 256 MB last-level cache, so it is timed warm (back to back) and
    scrubbed (a 512 MiB write between calls, timed on the forward's launches
    alone)."""
    from workloads import WORKLOADS, device_inputs

    w = WORKLOADS["fwd_f32"]
    B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
    q, k, v, _ = device_inputs(B, H, N, D, M, "f32", seed=0, scale=1.0 / D ** 0.5, device="cuda",
                               with_dout=False)
    out = torch.empty_like(v)
    plan = la.resolve_plan("forward", B, H, N, D, M, True, "f32")
    ws = torch.empty(max(1, la.workspace_bytes("forward", B, H, N, D, M, True, "f32")), dtype=torch.uint8,
                     device="cuda")

    def step():
        return la.forward(q, k, v, causal=True, out=out, workspace=ws)

    ms, prof, kname, avg_ms = timed_steps(la, torch, step, steps, warmup, settle=0.2)
    kernels = kernel_table(prof, 3, B, H, N, D, M, 4, plan["segments"], ceil)
    roof = step_roofline("fwd", B, H, N, D, M, 4, ms, kernels, TRAFFIC_FILE_F32, COUNTERS_FILE_F32,
                         "call: la_forward (every launch of the causal forward), warm")
    # scrubbed: a 512 MiB write evicts the inputs between calls; the forward's
    # own launches are timed with HIP events (the scrub is not)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        scrub.fill_(1)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms_cold = sorted(a.elapsed_time(b) for a, b in ev)[len(ev) // 2]
    del scrub
    alg = alg_bytes_per_ht("fwd", D, M, 4) * B * H * N
    log(f"fwd_f32: warm {ms:.4f} ms/call ({roof['frac']:.3f} of 8 TB/s), scrubbed median {ms_cold:.4f} ms; "
        f"breakdown {prof}")
    return {"metric": "fp32 causal linear-attn forward tokens/sec", "value": round(B * N / (ms / 1e3), 1),
            "unit": "tokens/s", "ms_per_call": round(ms, 4),
            "scrubbed": {"ms_per_call_median": round(ms_cold, 4),
                         "achieved_GBps": round(alg / (ms_cold / 1e3) / 1e9, 1),
                         "frac": round(alg / (ms_cold / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                         "note": "a 512 MiB device write before each call evicts the inputs from the caches"},
            "config": {"workload": "causal forward, fp32", "B": B, "H": H, "N": N, "D": D, "M": M, "plan": plan},
            "roofline": roof, "kernels": kernels}


COPY_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_fwdbwd_bf16.txt")
TRAFFIC_FILE_RET = os.path.join(PROFILES, "traffic_retention_fwdbwd_bf16.txt")
TRAFFIC_FILE_LONG = os.path.join(PROFILES, "traffic_long_bf16.txt")
TRAFFIC_FILE_F32 = os.path.join(PROFILES, "traffic_fwd_f32.txt")
TRAFFIC_FILE_DECODE = os.path.join(PROFILES, "traffic_decode_f32.txt")
COUNTERS_FILE = os.path.join(PROFILES, "counters_fwdbwd_bf16.txt")
COUNTERS_FILE_LONG = os.path.join(PROFILES, "counters_long_bf16.txt")
COUNTERS_FILE_F32 = os.path.join(PROFILES, "counters_fwd_f32.txt")

# HIP kernel symbols -> the library's launch names (la_profile_* names)
KERNEL_SYMBOLS = [
    ("k_bwd_fused_mfma", "mfma.bwd_fused"), ("k_fill_u32", "mfma.bwd_fused"), ("k_bwd_dkdv_mfma", "mfma.bwd_dkdv"), ("k_bwd_dq_mfma", "mfma.bwd_dq"), ("k_bwd_ragg_mfma", "mfma.bwd_dq"),
    ("k_fwd_f32mfma", "mfma.forward"), ("k_fwd_mfma_t128", "mfma.forward_t128"), ("k_fwd_mfma", "mfma.forward"), ("k_seg_state_wave64", "mfma.seg_state"),
    ("k_seg_state_f32mfma", "mfma.seg_state"), ("k_seg_state_mfma", "mfma.seg_state"), ("k_seg_scan", "seg_scan"),
    ("k_decode_vec", "decode"), ("k_ret_fwd_mfma", "ret.forward"), ("k_ret_seg_wave64", "ret.seg_state"),
    ("k_ret_seg_state", "ret.seg_state"), ("k_ret_scan", "ret.scan"), ("k_ret_dq", "ret.bwd_dq"),
    ("k_ret_rscan", "ret.rscan"), ("k_ret_dkdv", "ret.bwd_dkdv"), ("k_ret_dlg", "ret.dlg"),
]


def calibrate_copy(torch):
    """A plain device copy of exactly 1 GiB (read) + 1 GiB (write), repeated;
    run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to get the scale of
    those counters (bytes moved / counter value)."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "launches": 5}))


def kernel_source_sha():
    """Hash of the HIP sources: measured traffic is valid only for the
    kernels it was measured on."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kernelized_causal_attention_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_profile_table(path, cols=2):
    """A committed counter table (rows: launch name, then values per launch;
    a `source_sha` line; a `columns` line naming the value columns), or None
    when it is missing or was taken on different kernel sources.  cols=2:
    {name: (fetch bytes, write bytes)}; cols=None: {name: {column: value}}."""
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    sha = None
    names = None
    table = {}
    for line in lines:
        if line.startswith("source_sha"):
            sha = line.split()[1]
        elif line.startswith("columns"):
            names = line.split()[1:]
        elif line and not line.startswith("#"):
            parts = line.split()
            try:
                vals = [float(x) for x in parts[1:]]
            except ValueError:
                continue
            if cols == 2 and len(vals) >= 2:
                table[parts[0]] = (int(vals[0]), int(vals[1]))
            elif cols is None and names:
                table[parts[0]] = {n: x for n, x in zip(names, vals)}
    if sha != kernel_source_sha():
        return None
    return table


def measured_traffic(kname, path=TRAFFIC_FILE):
    """HBM bytes per launch of `kname` (FETCH_SIZE + WRITE_SIZE scaled by the
    copy calibration) from a committed table, or None."""
    t = read_profile_table(path)
    if t is None or kname not in t:
        return None
    return t[kname][0] + t[kname][1]


def launch_name(kernel_symbol):
    for sym, name in KERNEL_SYMBOLS:
        if kernel_symbol.startswith(sym):
            return name
    return None


def trace_summary(args):
    """Markdown table of the library's kernels in a rocprofv3 kernel trace:
    one row per kernel template instance and grid size (the grid tells the
    workloads apart), with durations in microseconds and the resources the
    trace records per dispatch (VGPRs, accumulation VGPRs, LDS bytes)."""
    import collections
    import csv
    import re

    rows = collections.defaultdict(list)
    res = {}
    for r in csv.DictReader(open(args.trace_summary)):
        m = re.search(r"(?<![A-Za-z0-9_])(k_[A-Za-z0-9_]+(<[^()]*>)?)", r["Kernel_Name"])
        if not m:
            continue
        key = (m.group(1), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]), int(r["Workgroup_Size_X"]))
        rows[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        res[key] = (r.get("VGPR_Count", ""), r.get("Accum_VGPR_Count", ""), r.get("LDS_Block_Size", ""))
    out = ["| kernel | workgroups x threads | calls | average (us) | min (us) | max (us) | VGPR | AGPR | LDS (bytes) |",
           "|---|---|---|---|---|---|---|---|---|"]
    for key in sorted(rows, key=lambda k: -sum(rows[k])):
        v = rows[key]
        vg, ag, lds = res[key]
        out.append(f"| {key[0]} | {key[1]} x {key[2]} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | "
                   f"{max(v):.1f} | {vg} | {ag} | {lds} |")
    print("\n".join(out))


def pmc_summary(args):
    """Per-kernel averages per dispatch of rocprofv3 --pmc counters.  Counter
    values of one dispatch are summed over their instances; FETCH_SIZE and
    WRITE_SIZE (KiB) are scaled to bytes by the calibration copy (bytes
    copied / counter bytes) when --pmc-calib is given.  Rows are keyed by the
    library's launch names (kernels of one launch name are summed per
    launch: e.g. the two kernels of the D = 128 dq sweep)."""
    import collections
    import csv
    import re

    def load(path):
        vals = collections.defaultdict(lambda: collections.defaultdict(float))  # (kernel, dispatch) -> counter
        for r in csv.DictReader(open(path)):
            m = re.search(r"(?<![A-Za-z0-9_])(k_[A-Za-z0-9_]+)", r["Kernel_Name"])
            sym = m.group(1) if m else r["Kernel_Name"].strip()[:60]
            vals[(sym, r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        return vals

    def calib(path, counter):
        # the copy kernel of --calibrate-copy moves COPY_BYTES per launch: the
        # dispatches with the largest counter value are those copies
        v = [d[counter] for d in load(path).values() if counter in d]
        v.sort()
        top = [x for x in v if x > 0.5 * v[-1]]
        return COPY_BYTES / (sum(top) / len(top) * 1024.0)

    factor = {}
    if args.pmc_calib:
        factor["FETCH_SIZE"] = calib(args.pmc_calib[0], "FETCH_SIZE")
        factor["WRITE_SIZE"] = calib(args.pmc_calib[1], "WRITE_SIZE")
    per = collections.defaultdict(lambda: collections.defaultdict(list))  # name -> counter -> per-launch values
    for path in args.pmc_summary:
        grouped = collections.defaultdict(lambda: collections.defaultdict(float))
        order = collections.defaultdict(list)
        for (sym, disp), d in load(path).items():
            name = launch_name(sym) or sym
            order[name].append((int(disp), sym, d))
        for name, lst in order.items():
            lst.sort()
            # consecutive dispatches of different symbols under one launch
            # name belong to one launch (they are issued back to back)
            syms = sorted({s for _, s, _ in lst})
            if len(syms) > 1:
                launches = [lst[i:i + len(syms)] for i in range(0, len(lst) - len(syms) + 1, len(syms))]
            else:
                launches = [[x] for x in lst]
            for launch in launches:
                tot = collections.defaultdict(float)
                for _, _, d in launch:
                    for c, x in d.items():
                        tot[c] += x
                for c, x in tot.items():
                    if c in ("FETCH_SIZE", "WRITE_SIZE"):
                        x = x * 1024.0 * factor.get(c, 1.0)
                    per[name][c].append(x)
    counters = sorted({c for d in per.values() for c in d})
    traffic = counters == ["FETCH_SIZE", "WRITE_SIZE"] or set(counters) <= {"FETCH_SIZE", "WRITE_SIZE"}
    out = []
    if args.pmc_title:
        out.append(f"# {args.pmc_title}")
    for c in args.pmc_command:
        out.append(f"#   {c}")
    if factor:
        out.append("# FETCH_SIZE / WRITE_SIZE scaled to bytes by the calibration copy (--calibrate-copy, "
                   f"{COPY_BYTES} bytes per launch): factors {factor.get('FETCH_SIZE', 1):.3f} / "
                   f"{factor.get('WRITE_SIZE', 1):.3f} bytes per counter byte")
    out.append("# values are averages per launch over every launch in the run")
    out.append(f"source_sha {kernel_source_sha()}")
    cols = ["FETCH_SIZE", "WRITE_SIZE"] if traffic else counters
    out.append("columns " + " ".join(cols) + " launches")
    for name in sorted(per):
        d = per[name]
        n = max(len(v) for v in d.values())
        row = [sum(d[c]) / len(d[c]) if d.get(c) else 0.0 for c in cols]
        out.append(f"{name:28s} " + " ".join(f"{x:16.6g}" if not traffic else f"{x:16.0f}" for x in row)
                   + f" {n:6d}")
    text = "\n".join(out) + "\n"
    if args.pmc_out:
        with open(args.pmc_out, "w") as f:
            f.write(text)
    print(text, end="")


def bench_decode(la, torch, steps):
    from workloads import WORKLOADS, decode_inputs

    w = WORKLOADS["decode_f32"]
    dev = "cuda"
    (pq, pk, pv), (sq, sk, sv) = decode_inputs(w, seed=0, device=dev)
    del pq
    S, Z = la.prefix_state(pk, pv)
    outs = torch.empty((steps, w.B, w.H, w.M), dtype=torch.float32, device=dev)
    for t in range(4):  # warm-up on scratch copies of the state
        la.decode_step(S.clone(), Z.clone(), sq[t], sk[t], sv[t])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    la.profile_enable(True, only="decode")
    e0.record(stream)
    for t in range(steps):
        la.decode_step(S, Z, sq[t % w.steps], sk[t % w.steps], sv[t % w.steps], out=outs[t])
    e1.record(stream)
    torch.cuda.synchronize()
    prof = la.profile_report()
    la.profile_enable(False)
    ms = e0.elapsed_time(e1)
    n, kms = prof.get("decode", (steps, ms))
    b = kernel_bytes("decode", w.B, w.H, 1, w.D, w.M, 4)
    kavg = kms / n
    gbs = b / (kavg / 1e3) / 1e9
    log(f"decode: {steps} steps in {ms:.2f} ms, kernel avg {kavg * 1e3:.1f} us, {gbs:.0f} GB/s")
    # The same steps captured once in a HIP graph and replayed: no host-side
    # launch work between consecutive steps (a serving loop's form).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(steps):
            la.decode_step(S, Z, sq[t % w.steps], sk[t % w.steps], sv[t % w.steps], out=outs[t])
    graph.replay()  # warm-up replay
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    gms = e0.elapsed_time(e1)
    del graph
    log(f"decode as one HIP graph: {steps} steps in {gms:.2f} ms ({gms / steps * 1e3:.1f} us/step)")
    # the softmax baseline on the same tokens: a KV cache filled with the
    # prefix, then the same steps (append, attend over every cached position)
    del S, Z
    cap = w.prefix + steps
    kc = torch.empty((w.B, w.H, cap, w.D), dtype=torch.float32, device=dev)
    vc = torch.empty((w.B, w.H, cap, w.M), dtype=torch.float32, device=dev)
    kc[:, :, :w.prefix] = pk
    vc[:, :, :w.prefix] = pv
    del pk, pv
    torch.cuda.synchronize()
    la.profile_enable(True, only="softmax.decode")
    e0.record(stream)
    for t in range(steps):
        la.softmax_decode_step(kc, vc, w.prefix + t, sq[t % w.steps], sk[t % w.steps], sv[t % w.steps], out=outs[t])
    e1.record(stream)
    torch.cuda.synchronize()
    sprof = la.profile_report()
    la.profile_enable(False)
    sms = e0.elapsed_time(e1)
    sn, skms = sprof.get("softmax.decode", (steps, sms))
    sb = sum(w.B * w.H * ((w.prefix + t + 1) * (w.D + w.M) * 4 + (2 * w.D + 2 * w.M) * 4) for t in range(steps))
    sgbs = sb / (skms / 1e3) / 1e9
    log(f"softmax KV-cache decode: {steps} steps in {sms:.2f} ms ({sms / steps * 1e3:.1f} us/step, cache "
        f"{w.prefix}..{w.prefix + steps - 1} tokens), {sgbs:.0f} GB/s; linear decode is {sms / ms:.1f}x faster")
    del kc, vc
    softmax = {"metric": "softmax KV-cache decode steps/sec", "value": round(steps / (sms / 1e3), 1),
               "unit": "steps/s", "avg_step_ms": round(sms / steps, 5),
               "cache_tokens": [w.prefix, w.prefix + steps - 1], "achieved_GBps": round(sgbs, 1),
               "frac": round(sgbs / PEAK_HBM_GBS, 4), "linear_decode_speedup": round(sms / ms, 2)}
    return {"metric": "decode steps/sec", "value": round(steps / (ms / 1e3), 1), "unit": "steps/s",
            "graph_replay": {"value": round(steps / (gms / 1e3), 1), "unit": "steps/s",
                             "avg_step_ms": round(gms / steps, 5),
                             "note": "the same steps captured once in a HIP graph, one replay timed"},
            "softmax_kv_cache": softmax,
            "config": {"workload": "batched RNN decode step, fp32 state", "B": w.B, "H": w.H, "D": w.D,
                       "M": w.M, "prefix": w.prefix, "steps": steps},
            "roofline": {"bound": "hbm", "kernel": "decode", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode", TRAFFIC_FILE_DECODE),
                         "alg_bytes_per_launch": b, "avg_launch_ms": round(kavg, 5)}}


def bench_retention(la, torch, steps, warmup):
    """Decayed / gated linear attention forward + backward on the same bf16
    shape as the main step (gates gamma_t ~ U(0.6, 1) per token; the
    backward reads the forward's segment states): tokens/s and the dominant
    kernel's HBM roofline."""
    from workloads import WORKLOADS, device_inputs

    w = WORKLOADS["fwdbwd_bf16"]
    B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
    dev = "cuda"
    q, k, v, g = device_inputs(B, H, N, D, M, "bf16", seed=1, scale=1.0 / D ** 0.5, device=dev)
    gen = torch.Generator(device=dev).manual_seed(2)
    lg = torch.log(torch.rand(B, H, N, device=dev, generator=gen) * 0.4 + 0.6)
    ws_f = torch.empty(max(1, la.workspace_bytes("retention_forward", B, H, N, D, M, True, "bf16")),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, la.workspace_bytes("retention_backward", B, H, N, D, M, True, "bf16")),
                       dtype=torch.uint8, device=dev)
    plan_f = la.resolve_plan("retention_forward", B, H, N, D, M, True, "bf16")
    plan_b = la.resolve_plan("retention_backward", B, H, N, D, M, True, "bf16")
    saved = torch.empty(la.retention_saved_bytes(B, H, N, D, M), dtype=torch.uint8, device=dev)

    def step():
        la.retention_forward(q, k, v, lg, workspace=ws_f, saved=saved)
        return la.retention_backward(q, k, v, lg, g, workspace=ws_b, saved=saved)

    for _ in range(warmup + 3):
        step()
    torch.cuda.synchronize()
    la.profile_enable(True)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    prof = la.profile_report()
    kname = max(prof.items(), key=lambda kv: kv[1][1])[0]
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    la.profile_enable(True, only=kname)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    nl, tot_ms = la.profile_report()[kname]
    la.profile_enable(False)
    ms = e0.elapsed_time(e1) / steps
    kernels = {}
    for name, (n, t) in sorted(prof.items()):
        P = plan_b["segments"] if name in ("ret.bwd_dq", "ret.rscan", "ret.bwd_dkdv", "ret.dlg") else plan_f["segments"]
        b = kernel_bytes(name, B, H, N, D, M, 2, P)
        avg = t / n
        kernels[name] = {"launches_per_step": n / 3, "avg_ms": round(avg, 4), "alg_bytes": b,
                         "GBps": round(b / (avg / 1e3) / 1e9, 1) if b else None}
    avg_ms = tot_ms / nl
    kb = kernels[kname]["alg_bytes"]
    gbs = kb / (avg_ms / 1e3) / 1e9
    log(f"retention: {ms:.3f} ms/step, {B * N / (ms / 1e3):.4g} tokens/s; dominant {kname} {avg_ms:.4f} ms "
        f"{gbs:.0f} GB/s; breakdown {prof}")
    return {"metric": "decayed linear-attn (retention) fwd+bwd tokens/sec", "value": round(B * N / (ms / 1e3), 1),
            "unit": "tokens/s", "ms_per_step": round(ms, 4),
            "config": {"workload": "retention forward+backward, bf16 in / fp32 accumulate, gamma_t ~ U(0.6, 1)",
                       "B": B, "H": H, "N": N, "D": D, "M": M, "plan_forward": plan_f, "plan_backward": plan_b},
            "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(kname, TRAFFIC_FILE_RET),
                         "alg_bytes_per_launch": kb, "avg_launch_ms": round(avg_ms, 4)},
            "kernels": kernels}


def bench_poly(la, torch, steps, warmup):
    """Degree-2 polynomial-kernel attention forward + backward on the same
    bf16 shape as the main step: tokens/s and the dominant kernel's MFMA
    roofline (matrix-product flops over its time, against the dense bf16
    peak)."""
    from workloads import WORKLOADS, device_inputs

    w = WORKLOADS["fwdbwd_bf16"]
    B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
    dev = "cuda"
    q, k, v, g = device_inputs(B, H, N, D, M, "bf16", seed=3, scale=1.0 / D ** 0.5, device=dev)
    out = torch.empty((B, H, N, M), dtype=torch.bfloat16, device=dev)
    den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, la.workspace_bytes("poly_backward", B, H, N, D, M, True, "bf16")), dtype=torch.uint8,
                     device=dev)

    def step():
        la.poly_forward(q, k, v, out=out, den=den)
        return la.poly_backward(q, k, v, out, g, den, workspace=ws)

    for _ in range(warmup + 3):
        step()
    torch.cuda.synchronize()
    la.profile_enable(True)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    prof = la.profile_report()
    kname = max(prof.items(), key=lambda kv: kv[1][1])[0]
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    la.profile_enable(True, only=kname)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    nl, tot_ms = la.profile_report()[kname]
    la.profile_enable(False)
    ms = e0.elapsed_time(e1) / steps
    kernels = {}
    for name, (n, t) in sorted(prof.items()):
        f = kernel_flops(name, B, H, N, D, M)
        avg = t / n
        kernels[name] = {"launches_per_step": n / 3, "avg_ms": round(avg, 4), "flops": f,
                         "TFLOPs": round(f / (avg / 1e3) / 1e12, 1)}
    avg_ms = tot_ms / nl
    kf = kernels[kname]["flops"]
    tf = kf / (avg_ms / 1e3) / 1e12
    step_tf = sum(v["flops"] for v in kernels.values()) / (ms / 1e3) / 1e12
    log(f"poly: {ms:.3f} ms/step, {B * N / (ms / 1e3):.4g} tokens/s, {step_tf:.0f} TFLOP/s over the step; dominant "
        f"{kname} {avg_ms:.4f} ms {tf:.0f} TFLOP/s; breakdown {prof}")
    return {"metric": "polynomial-kernel (degree-2) causal attention fwd+bwd tokens/sec",
            "value": round(B * N / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
            "step_tflops": round(step_tf, 1),
            "config": {"workload": "(q.k)^2 causal attention forward+backward, bf16 in / fp32 accumulate",
                       "B": B, "H": H, "N": N, "D": D, "M": M},
            "roofline": with_mfma_ceiling(
                {"bound": "mfma", "kernel": kname, "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                 "flops_per_launch": kf, "avg_launch_ms": round(avg_ms, 4)}),
            "kernels": kernels, "decode": bench_poly_decode(la, torch), "crossover": bench_poly_crossover(la, torch)}


def bench_poly_crossover(la, torch, B=1, H=16, D=64, M=64):
    """The degree-2 map's two evaluation orders across sequence lengths (the
    walkthrough's section 2, 'feature map and computation cost', item (3):
    the linear form costs N D^2 M, the masked sum N^2 D, so the linear form
    wins once N is large against D^2).  Timed per call on 16 heads: the
    masked-sum causal forward (la_poly_forward) and the linear form's state
    accumulation S = phi(K)^T V over the D^2 features (la_poly_prefix_state);
    a causal linear-form forward does that accumulation plus a read-out of
    the same flop count (phi(Q_i)^T S_i), so twice the accumulation's time
    stands for it (a chunked linear-form forward is not built)."""
    from workloads import device_inputs

    rows = []
    cross = None
    for N in (1024, 2048, 4096, 8192, 16384, 32768):
        q, k, v, _ = device_inputs(B, H, N, D, M, "bf16", seed=6, scale=1.0 / D ** 0.5, device="cuda",
                                   with_dout=False)
        out = torch.empty_like(v)

        def tm(fn, n=5):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        ms_masked = tm(lambda: la.poly_forward(q, k, v, out=out))
        ms_state = tm(lambda: la.poly_prefix_state(k, v))
        rows.append({"N": N, "masked_sum_ms": round(ms_masked, 4), "linear_state_ms": round(ms_state, 4),
                     "linear_form_estimate_ms": round(2 * ms_state, 4)})
        if cross is None and ms_masked > 2 * ms_state:
            cross = N
        del q, k, v, out
    log("poly crossover: " + ", ".join(f"N={r['N']} masked {r['masked_sum_ms']:.3f} ms vs linear ~"
                                       f"{r['linear_form_estimate_ms']:.3f} ms" for r in rows))
    return {"config": {"B": B, "H": H, "D": D, "M": M, "dtype": "bf16"}, "rows": rows,
            "first_N_where_linear_form_is_faster": cross,
            "flop_crossover_N": 4 * D * D * M // (D + M),
            "note": "linear form = 2 x the D^2-feature state accumulation (update + read-out of equal flops); the "
                    "pages put the crossover at N > D^2 = %d; counting the causal constants, at 4 D^2 M / (D + M)"
                    % (D * D)}


def bench_softmax(la, torch, steps, warmup):
    """The softmax baseline's causal forward on the main step's shape against
    the linear-attention forward on the same inputs (the pages' speed claim
    as a kernel ratio on one GPU)."""
    from workloads import WORKLOADS, device_inputs

    w = WORKLOADS["fwdbwd_bf16"]
    B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
    q, k, v, _ = device_inputs(B, H, N, D, M, "bf16", seed=5, scale=1.0 / D ** 0.5, device="cuda")
    out = torch.empty((B, H, N, M), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, la.workspace_bytes("forward", B, H, N, D, M, True, "bf16")), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(warmup + 3):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    sm_ms = timed(lambda: la.softmax_forward(q, k, v, out=out))
    la_ms = timed(lambda: la.forward(q, k, v, causal=True, out=out, workspace=ws))
    flops = B * H * (N * (N + 1) // 2) * (2 * D + 2 * M)
    tf = flops / (sm_ms / 1e3) / 1e12
    log(f"softmax forward: {sm_ms:.3f} ms ({tf:.0f} TFLOP/s); linear-attention forward {la_ms:.3f} ms "
        f"({sm_ms / la_ms:.1f}x)")
    return {"metric": "softmax causal attention forward tokens/sec", "value": round(B * N / (sm_ms / 1e3), 1),
            "unit": "tokens/s", "ms": round(sm_ms, 4),
            "config": {"workload": "softmax(QK^T/sqrt(D))V causal forward, bf16 in / fp32 accumulate", "B": B,
                       "H": H, "N": N, "D": D, "M": M},
            "roofline": with_mfma_ceiling(
                {"bound": "mfma", "kernel": "softmax.forward", "achieved": round(tf, 1),
                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                 "traffic": None, "flops_per_launch": flops, "avg_launch_ms": round(sm_ms, 4)}),
            "linear_forward_ms": round(la_ms, 4), "linear_forward_speedup": round(sm_ms / la_ms, 2),
            "speedup_caveat": f"ratio against this library's online-softmax forward, which runs at "
                              f"{tf / PEAK_BF16_TFLOPS:.2f} of the dense bf16 MFMA peak; at the full peak the "
                              f"softmax forward would take {flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3:.3f} ms, "
                              f"a ratio of {flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3 / la_ms:.2f}",
            "speedup_at_softmax_peak": round(flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3 / la_ms, 2)}


def bench_poly_decode(la, torch, steps=256, B=16, H=32, D=64, M=64, prefix=512):
    """The polynomial map's recurrent decode step (the linear form: a
    D^2 x M fp32 state per head, 1 MB at D = M = 64) after a bf16 prefix:
    steps/s and HBM GB/s."""
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(4)
    pk = (torch.randn(B, H, prefix, D, device=dev, generator=gen) / D ** 0.5).to(torch.bfloat16)
    pv = (torch.randn(B, H, prefix, M, device=dev, generator=gen) / D ** 0.5).to(torch.bfloat16)
    S, Z = la.poly_prefix_state(pk, pv)
    sq, sk, sv = ((torch.randn(steps, B, H, n, device=dev, generator=gen) / D ** 0.5).to(torch.bfloat16)
                  for n in (D, D, M))
    outs = torch.empty((steps, B, H, M), dtype=torch.bfloat16, device=dev)
    for t in range(4):
        la.poly_decode_step(S.clone(), Z.clone(), sq[t], sk[t], sv[t])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    la.profile_enable(True, only="poly.decode")
    e0.record(stream)
    for t in range(steps):
        la.poly_decode_step(S, Z, sq[t], sk[t], sv[t], out=outs[t])
    e1.record(stream)
    torch.cuda.synchronize()
    n, kms = la.profile_report().get("poly.decode", (steps, e0.elapsed_time(e1)))
    la.profile_enable(False)
    ms = e0.elapsed_time(e1)
    C = D * D
    b = B * H * (2 * C * M * 4 + 2 * C * 4 + 2 * (2 * D + M) + 2 * M)
    kavg = kms / n
    gbs = b / (kavg / 1e3) / 1e9
    log(f"poly decode: {steps} steps in {ms:.2f} ms, kernel avg {kavg * 1e3:.1f} us, {gbs:.0f} GB/s")
    return {"metric": "polynomial-map decode steps/sec", "value": round(steps / (ms / 1e3), 1), "unit": "steps/s",
            "config": {"workload": "degree-2 polynomial map recurrent decode step, fp32 D^2 x M state, bf16 tokens",
                       "B": B, "H": H, "D": D, "M": M, "prefix": prefix, "steps": steps},
            "roofline": {"bound": "hbm", "kernel": "poly.decode", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                         "alg_bytes_per_launch": b, "avg_launch_ms": round(kavg, 5)}}


# ------------------------------------------------------ oracle baseline ----
# The fp64 oracle (test infrastructure; timed here only) on the host's cores:
# a pool of single-threaded worker processes, one task per head (or per
# block of decode heads).  Each task draws its own inputs with the workloads'
# recipe (seeded per head; the timing does not depend on the values) and
# times only the oracle call.
def _oracle_task(task):
    import numpy as np

    import oracle

    kind, seed, idx, N, D, M, extra = task
    rng = np.random.default_rng([seed, idx])
    s = 1.0 / np.sqrt(D)
    if kind == "fwdbwd":  # the oracle's backward runs the forward recurrence and both sweeps
        q, k, v = (rng.standard_normal((1, N, n)) * s for n in (D, D, M))
        g = rng.standard_normal((1, N, M))
        t0 = time.perf_counter()
        oracle.backward(q, k, v, g, True)
        return time.perf_counter() - t0
    if kind == "fwd":
        q, k, v = (rng.standard_normal((1, N, n)) * s for n in (D, D, M))
        t0 = time.perf_counter()
        oracle.forward_recurrent(q, k, v, True)
        return time.perf_counter() - t0
    if kind == "decode":  # `idx`-th block of `extra[0]` heads, `extra[1]` steps after a prefix of N tokens
        nh, steps = extra
        pk, pv = rng.standard_normal((nh, N, D)) * s, rng.standard_normal((nh, N, M)) * s
        S, Z = oracle.prefix_state(pk, pv)
        del pk, pv
        qs, ks = rng.standard_normal((steps, nh, D)) * s, rng.standard_normal((steps, nh, D)) * s
        vs = rng.standard_normal((steps, nh, M)) * s
        t0 = time.perf_counter()
        oracle.decode_steps(S, Z, qs, ks, vs)
        return time.perf_counter() - t0
    raise ValueError(kind)


def cpu_baseline(workers=0):
    """Time the oracle on the host cores before any GPU work: the headline
    fwd+bwd workload on all 128 heads, the long-sequence forward on all 16
    heads and 8 decode steps on all 8192 heads."""
    import multiprocessing as mp

    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    k = workers if workers > 0 else max(1, min(avail, 16))
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    saved_env = {n: os.environ.get(n) for n in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for n in saved_env:
        os.environ[n] = "1"  # one thread per worker process (inherited at spawn)
    ctx = mp.get_context("spawn")
    res = {}
    try:
        with ctx.Pool(k) as pool:
            pool.map(_oracle_task, [("fwdbwd", 0, i, 256, 64, 64, None) for i in range(k)])  # warm the workers
            for key, tasks in (
                    ("fwdbwd_bf16", [("fwdbwd", 0, i, 8192, 64, 64, None) for i in range(128)]),
                    ("long_bf16", [("fwd", 1, i, 65536, 128, 128, None) for i in range(16)]),
                    ("decode_f32", [("decode", 2, i, 512, 128, 128, (128, 8)) for i in range(64)])):
                t0 = time.perf_counter()
                times = pool.map(_oracle_task, tasks, chunksize=1)
                wall = time.perf_counter() - t0
                res[key] = (wall, sum(times), len(tasks))
                log(f"cpu oracle {key}: {len(tasks)} tasks on {k} workers, wall {wall:.2f} s "
                    f"(oracle time {sum(times):.1f} s)")
    finally:
        for n, x in saved_env.items():
            if x is None:
                os.environ.pop(n, None)
            else:
                os.environ[n] = x
    wall, busy, n = res["fwdbwd_bf16"]
    tokens = 8 * 8192  # B * N of the whole batch (128 heads)
    lw, lbusy, _ = res["long_bf16"]
    dw, dbusy, _ = res["decode_f32"]
    return {"value": round(tokens / wall, 1), "unit": "tokens/s", "cores": k, "kind": "oracle",
            "sample": f"fp64 numpy oracle backward (forward recurrence + both gradient sweeps) on all 128 heads "
                      f"of the 8x16x8192, D=M=64 workload (inputs drawn per head with the same recipe), one "
                      f"head per task on {k} single-threaded worker processes: wall {wall:.2f} s, "
                      f"{busy:.1f} s of oracle time",
            "cpu": cpu, "cores_available": avail,
            "long_bf16": {"value": round(65536 / lw, 1), "unit": "tokens/s",
                          "sample": f"forward recurrence on all 16 heads of 1x16x65536, D=M=128, wall {lw:.2f} s "
                                    f"({lbusy:.1f} s of oracle time)"},
            "decode_f32": {"value": round(8 / (dbusy / k), 2), "unit": "steps/s",
                           "sample": f"8 decode steps on all 8192 heads (256x32, D=M=128) in 64 blocks of 128 "
                                     f"heads, each after its own 512-token prefix (not timed): {dbusy:.2f} s of "
                                     f"oracle time, spread over the {k} workers (wall {dw:.2f} s including "
                                     f"the prefixes)"}}


if __name__ == "__main__":
    main()
