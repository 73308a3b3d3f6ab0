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
  roofline      -- the dominant kernel's algorithmic bytes per launch over its
                   average launch time (HIP events around every launch inside
                   the timed region), against 8 TB/s.
  cpu_baseline  -- the fp64 oracle (test infrastructure, timed here only) on a
                   bounded sample of the same workload's heads, scaled to
                   tokens/s of the whole batch.
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


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the decode measurement")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
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
    return ap.parse_args()


CEILING_EXE = os.path.join(ROOT, "kernelized_causal_attention_amd", "_lib", "hbm_ceiling")
# the traffic mix of each kernel (tensors read / written), for its practical ceiling
KERNEL_MIX = {"mfma.seg_state": "r2", "mfma.forward": "r3w1", "mfma.bwd_dq": "r4w1", "mfma.bwd_dkdv": "r4w2",
              "decode": "r1w1"}


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
        mixes[d["mix"]] = d["GBps"]
    log("streaming ceilings (GB/s): " + ", ".join(f"{k} {v:.0f}" for k, v in mixes.items()))
    return mixes


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
    if family == "mfma" and base == "bwd_dkdv":
        # reads q, k, v, dout and (c, den); writes dk, dv
        return ht * (es * (2 * D + 2 * M) + 8 + es * (D + M))
    if base == "forward":
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(every (b,h) head is independent; multi-GPU sharding is described in the design notes, "
              "not run).", file=sys.stderr)
        sys.exit(2)
    if args.ceilings:
        r = subprocess.run([CEILING_EXE])
        sys.exit(r.returncode)
    ceil = None
    if not (args.no_ceiling or args.calibrate_copy or args.retention_only or args.poly_only):
        ceil = hbm_ceilings()

    import torch

    if args.calibrate_copy:
        calibrate_copy(torch)
        return

    import kernelized_causal_attention_amd as la
    from workloads import WORKLOADS, device_inputs

    if args.retention_only:
        torch.cuda.set_device(0)
        print(json.dumps(bench_retention(la, torch, args.steps, args.warmup)), flush=True)
        return
    if args.poly_only:
        torch.cuda.set_device(0)
        print(json.dumps(bench_poly(la, torch, args.steps, args.warmup)), flush=True)
        return

    w = WORKLOADS["fwdbwd_bf16"]
    B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
    es = 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
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
    # Untimed settling: an idle GPU needs a few hundred milliseconds of load
    # to reach its steady clocks (the first ~0.3 s of steps run ~5% slower).
    t_settle = time.time() + args.settle
    while time.time() < t_settle:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # A short pass with every kernel timed: the per-kernel breakdown, and
    # which kernel dominates.
    nbreak = 3
    la.profile_enable(True)
    for _ in range(nbreak):
        step()
    torch.cuda.synchronize()
    prof = la.profile_report()
    kname = max(prof.items(), key=lambda kv: kv[1][1])[0]

    # Timed region: exactly K steps between synchronisations; only the
    # dominant kernel is bracketed by events (on the stream it runs on).
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    la.profile_enable(True, only=kname)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    nl, tot_ms = la.profile_report()[kname]
    la.profile_enable(False)
    ms = t0.elapsed_time(t1) / args.steps
    tokens = B * N
    value = tokens / (ms / 1e3)
    log(f"{ms:.3f} ms/step, {value:.4g} tokens/s; dominant {kname} {tot_ms / nl:.4f} ms; "
        f"breakdown: {prof}")
    P = plan_b["segments"] if "bwd" in kname or "scan" in kname else plan_f["segments"]
    kb = kernel_bytes(kname, B, H, N, D, M, es, P)
    avg_ms = tot_ms / nl
    achieved = kb / (avg_ms / 1e3) / 1e9
    kernels = {}
    for name, (n, t) in sorted(prof.items()):
        b = kernel_bytes(name, B, H, N, D, M, es, P)
        avg = t / n
        kernels[name] = {"launches_per_step": n / nbreak, "avg_ms": round(avg, 4),
                         "alg_bytes": b, "GBps": round(b / (avg / 1e3) / 1e9, 1) if b else None}
        mix = KERNEL_MIX.get(name)
        if ceil and mix in ceil and b:
            kernels[name]["ceiling_mix"] = mix
            kernels[name]["frac_of_ceiling"] = round(b / (avg / 1e3) / 1e9 / ceil[mix], 4)
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
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(kname),
                     "alg_bytes_per_launch": kb, "avg_launch_ms": round(avg_ms, 4)},
        "kernels": kernels,
    }
    if ceil:
        mix = KERNEL_MIX.get(kname)
        result["hbm_ceiling"] = {
            "source": "streaming microbenchmark on this GPU (kernelized_causal_attention_amd/_lib/hbm_ceiling): "
                      "plain 16-byte-vector kernels over 134 MB tensors, GB/s per traffic mix",
            "mixes": ceil, "dominant_mix": mix,
            "dominant_frac_of_ceiling": round(achieved / ceil[mix], 4) if mix in ceil else None}

    if not args.no_extra:
        result["decode"] = bench_decode(la, torch, args.decode_steps)
        if ceil and "r1w1" in ceil:
            result["decode"]["roofline"]["frac_of_ceiling"] = round(
                result["decode"]["roofline"]["achieved"] / ceil["r1w1"], 4)
        result["retention"] = bench_retention(la, torch, args.steps, args.warmup)
        result["poly"] = bench_poly(la, torch, args.steps, args.warmup)
        result["softmax"] = bench_softmax(la, torch, args.steps, args.warmup)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(q, k, v, g, B, H, N, args.cpu_seconds)

    print(json.dumps(result), flush=True)


COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwdbwd_bf16.txt")
TRAFFIC_FILE_RET = os.path.join(ROOT, "profiles", "traffic_retention_fwdbwd_bf16.txt")


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


def measured_traffic(kname, path=TRAFFIC_FILE):
    """HBM bytes per launch of `kname` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or
    None when it is missing or was taken on different kernel sources."""
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    sha = None
    table = {}
    for line in lines:
        if line.startswith("source_sha"):
            sha = line.split()[1]
        elif line and not line.startswith("#"):
            parts = line.split()
            if len(parts) >= 3:
                try:
                    table[parts[0]] = int(float(parts[1])) + int(float(parts[2]))
                except ValueError:
                    pass
    if sha != kernel_source_sha():
        return None
    return table.get(kname)


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
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
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
            "roofline": {"bound": "mfma", "kernel": kname, "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                         "flops_per_launch": kf, "avg_launch_ms": round(avg_ms, 4)},
            "kernels": kernels, "decode": bench_poly_decode(la, torch)}


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
            "roofline": {"bound": "mfma", "kernel": "softmax.forward", "achieved": round(tf, 1),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": None, "flops_per_launch": flops, "avg_launch_ms": round(sm_ms, 4)},
            "linear_forward_ms": round(la_ms, 4), "linear_forward_speedup": round(sm_ms / la_ms, 2)}


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


def cpu_baseline(q, k, v, g, B, H, N, budget_s):
    """Time the fp64 oracle's backward (which runs the forward recurrence
    and both gradient sweeps) on a sample of heads, single-threaded."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    def host(t, sel):
        return t[sel].detach().float().cpu().numpy().astype(np.float64)

    heads = [(b, h) for b in range(B) for h in range(H)]

    def run(n):
        sel = (np.array([b for b, _ in heads[:n]]), np.array([h for _, h in heads[:n]]))
        qq, kk, vv, gg = (host(t, sel) for t in (q, k, v, g))
        with threadpool_limits(1):
            t0 = time.perf_counter()
            oracle.backward(qq, kk, vv, gg, True)
            return time.perf_counter() - t0

    t_probe = run(2)
    n = int(min(len(heads), max(2, 2 * budget_s / max(t_probe, 1e-3))))
    t = run(n) if n > 2 else t_probe
    tokens_per_s = n * N / (H * t)
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    log(f"cpu oracle: {n} heads x {N} tokens in {t:.2f} s -> {tokens_per_s:.4g} tokens/s")
    return {"value": round(tokens_per_s, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"fp64 numpy oracle backward (forward recurrence + both gradient sweeps) on {n} of "
                      f"{B * H} heads at full N={N}, {t:.2f} s, single thread; scaled to the batch as "
                      f"n*N/(H*t)", "cpu": cpu}


if __name__ == "__main__":
    main()
