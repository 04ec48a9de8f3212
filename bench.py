#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one causal forward pass (fa_fwd) over the workload B4 H32 N4096
D128 bf16 (iid N(0,1) inputs, scale 1/sqrt(128)), inputs resident in HBM.
Prints ONE JSON line with the throughput in TFLOP/s, the roofline position of
the forward kernel, the backward pass (fa_bwd, B2 H32 N4096 D128 causal)
against the same roofline, the decoding-shaped forward (fa_fwd_splitkv, one
query against a 16384-token cache, B8 H32 D128) against HBM bandwidth, the
varlen (16 packed causal sequences) and long-context (B1 H32 N65536)
forwards, the varlen backward (fa_bwd_varlen), chunked prefill (fa_fwd_qk),
the fp16 forward, dropout forward and backward, the metric workload with
L2/MALL flushed before each launch, and
the fp64 CPU oracle timed on a bounded sample of the same workload.

FLOP convention: 4*D flops per (query, key) pair, causal counted as half of
B*H*N^2 pairs; backward counted as 2.5x forward; softmax work not counted.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s & % bf16 MFMA peak, causal B4 H32 N4096 D128"
# MI355X dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU
PEAK_BF16_TFLOPS = 2516.6
HBM_GBS = 8000.0  # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_kernel_causal_b4h32n4096d128_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_io_aware_44_amd", "csrc", f)
                  for f in ("fa_fwd.hip", "fa_device.hpp", "fa_schedule.hpp")]


def log(*a):
    print("bench:", *a, file=sys.stderr, flush=True)


def fwd_flops(B, H, N, D, causal):
    return 4.0 * B * H * N * N * D * (0.5 if causal else 1.0)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary, or None when absent or taken on different kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    src = re.search(r"^source_hash:\s*(\S+)", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def time_launches(torch, fn, steps, warmup):
    """Warm up, then time exactly `steps` calls: whole-region elapsed time
    and per-launch durations, all with HIP events on the launch stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s, e in ev:
        s.record()
        fn()
        e.record()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    per = [s.elapsed_time(e) for s, e in ev]
    return total, per


def cpu_baseline(budget_s: float):
    """The fp64 oracle, untuned, on whole (batch, head) slices of the causal
    workload, taken in order until about budget_s seconds of CPU work."""
    import attn_inputs as ai
    import oracle
    w = ai.CAUSAL
    q, k, v = ai.qkv(w.B, w.H, w.N, w.D, w.seed)
    per_head = fwd_flops(1, 1, w.N, w.D, True)
    done, elapsed = 0, 0.0
    for bh in range(w.B * w.H):
        b, h = divmod(bh, w.H)
        args = [x[b, h][None, None].double().numpy() for x in (q, k, v)]
        t = time.perf_counter()
        oracle.fwd(*args, w.scale, True)
        elapsed += time.perf_counter() - t
        done += 1
        if elapsed >= budget_s:
            break
    return {
        "value": per_head * done / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "%d of %d (batch, head) slices of causal B4 H32 N4096 D128, "
                  "every row, fp64, %.1f s" % (done, w.B * w.H, elapsed),
    }


def run_backward(torch, ai, fa, steps):
    """fa_bwd on causal B2 H32 N4096 D128 (O and L from fa_fwd)."""
    wb = ai.BACKWARD
    log("backward", wb.name)
    qb, kb, vb, dob = (x.cuda() for x in ai.backward_inputs())
    ob, lseb = fa.fa_fwd(qb, kb, vb, softmax_scale=wb.scale, causal=True)
    dq, dk, dv = (torch.empty_like(qb) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_size(wb.B, wb.H, wb.N, wb.D),
                     dtype=torch.uint8, device="cuda")

    def bwd_step():
        fa.fa_bwd(qb, kb, vb, ob, lseb, dob, softmax_scale=wb.scale, causal=True,
                  dq=dq, dk=dk, dv=dv, workspace=ws)

    # about 30 ms of warm-up: the clocks ramp after the host-side input work
    btotal, bper = time_launches(torch, bwd_step, steps, 30)
    bflops = 2.5 * fwd_flops(wb.B, wb.H, wb.N, wb.D, True)
    b_ms = btotal / steps
    backward = {"workload": wb.name, "ms": round(b_ms, 4),
                "tflops": round(bflops / (b_ms * 1e-3) / 1e12, 2),
                "frac": round(bflops / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "flops_per_call": bflops, "launches": 3,
                # per call (HIP events around each call's three launches)
                "calls": launch_stats(wb.name, bflops, bper)}
    del qb, kb, vb, dob, ob, lseb, dq, dk, dv, ws
    return backward


def run_decode(torch, ai, fa, steps):
    """fa_fwd_splitkv on one new query per sequence against a 16384-token
    cache (B8 H32 D128): HBM-bound, so reported as bytes per second."""
    B, H, Nq, Nk, D = 8, 32, 1, 16384, 128
    log("decode B%d H%d Nq%d Nk%d D%d" % (B, H, Nq, Nk, D))
    q = ai.randn_bf16((B, H, Nq, D), 900).cuda()
    k = ai.randn_bf16((B, H, Nk, D), 901).cuda()
    v = ai.randn_bf16((B, H, Nk, D), 902).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    ws_bytes = fa.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")

    def step():
        fa.fa_fwd_splitkv(q, k, v, causal=True, out=o, lse=lse, workspace=ws)

    total, _ = time_launches(torch, step, steps, 80)  # about 30 ms of warm-up
    ms = total / steps
    # algorithmic bytes: K and V read once, Q read and O, L written once
    nbytes = 2 * B * H * Nk * D * 2 + 2 * B * H * Nq * D * 2 + B * H * Nq * 4
    return {"workload": "decode B%d H%d Nq%d Nk%d D%d (fa_fwd_splitkv)"
                        % (B, H, Nq, Nk, D),
            "ms": round(ms, 4), "bound": "hbm", "unit": "GB/s",
            "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": HBM_GBS,
            "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_GBS, 4),
            "bytes_per_call": nbytes,
            # one launch when each head's keys form one range, else the
            # ranges' launch and the merge
            "launches": 2 if ws_bytes else 1}


def gpu_randn_bf16(torch, shape, seed):
    """Seeded iid N(0,1) fp32 drawn on the GPU, rounded to bf16 (timing-only
    inputs: same shape and distribution as the parity inputs, generated
    where they are used)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def run_other_configs(torch, ai, fa, steps):
    """The varlen forward and backward and the long-context forward
    workloads, same roofline."""
    out = {}
    # varlen: 16 causal sequences, lengths U[128, 8192], packed [H, total, D]
    lengths = ai.varlen_lengths(ai.VARLEN_LENGTH_SEED)
    cu = ai.cu_seqlens(lengths).cuda()
    total, H, D = int(sum(lengths)), ai.VARLEN_H, ai.VARLEN_D
    log("varlen: %d sequences, %d tokens" % (len(lengths), total))
    q, k, v = (gpu_randn_bf16(torch, (H, total, D), ai.VARLEN_DATA_SEED * 10 + i)
               for i in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device="cuda")
    scale = ai.default_scale(D)

    def vstep():
        fa.fa_fwd_varlen(q, k, v, cu, max(lengths), softmax_scale=scale, causal=True,
                         out=o, lse=lse)

    _, per = time_launches(torch, vstep, steps, 10)
    flops = sum(4.0 * H * D * n * n * 0.5 for n in lengths)
    out["varlen"] = launch_stats(ai.VARLEN_NAME, flops, per)
    # the packed backward on the same workload (three launches per call;
    # counted as 2.5x the forward's flops)
    do = gpu_randn_bf16(torch, (H, total, D), ai.VARLEN_DATA_SEED * 10 + 3)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_size(1, H, total, D), dtype=torch.uint8,
                     device="cuda")

    def vbstep():
        fa.fa_bwd_varlen(q, k, v, o, lse, do, cu, max(lengths), softmax_scale=scale,
                         causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)

    _, per = time_launches(torch, vbstep, steps, 3)
    out["varlen_backward"] = launch_stats("varlen causal bwd 16 seqs U[128,8192] H32 D128",
                                          2.5 * flops, per)
    del q, k, v, o, lse, do, dq, dk, dv, ws
    # long context: B1 H32 N65536 D128 causal
    w = ai.LONG
    log("long:", w.name)
    q, k, v = (gpu_randn_bf16(torch, (w.B, w.H, w.N, w.D), w.seed * 10 + i) for i in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")

    def lstep():
        fa.fa_fwd(q, k, v, softmax_scale=w.scale, causal=True, out=o, lse=lse)

    _, per = time_launches(torch, lstep, max(2, steps // 2), 1)
    out["long"] = launch_stats(w.name, fwd_flops(w.B, w.H, w.N, w.D, True), per)
    del q, k, v, o, lse
    return out


def run_next_rows(torch, ai, fa, steps):
    """The widened entry points on shapes of their own, same roofline:
    chunked prefill (fa_fwd_qk: 4096 new queries against a 16384-key cache,
    causal mask aligned bottom-right), the fp16 twin of the metric forward,
    and attention dropout (p = 0.1) forward and backward on the backward's
    shape.  Dropout's flops are counted as without it (the generator's work
    is not counted)."""
    out = {}
    B, H, Nq, Nk, D = 1, 32, 4096, 16384, 128
    log("chunked prefill: B%d H%d Nq%d Nk%d D%d" % (B, H, Nq, Nk, D))
    q = gpu_randn_bf16(torch, (B, H, Nq, D), 7000)
    k, v = (gpu_randn_bf16(torch, (B, H, Nk, D), 7001 + i) for i in range(2))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    scale = ai.default_scale(D)

    def qkstep():
        fa.fa_fwd_qk(q, k, v, softmax_scale=scale, causal=True, out=o, lse=lse)

    _, per = time_launches(torch, qkstep, steps, 10)
    pairs = Nq * (Nk - Nq) + Nq * (Nq + 1) / 2  # query i reads keys 0 .. i + Nk - Nq
    out["chunked_prefill"] = launch_stats(
        "chunked prefill B1 H32 Nq4096 Nk16384 D128 causal (fa_fwd_qk)", 4.0 * D * B * H * pairs,
        per)
    del q, k, v, o, lse
    w = ai.CAUSAL
    log("fp16:", w.name)
    q, k, v = (gpu_randn_bf16(torch, (w.B, w.H, w.N, w.D), w.seed * 10 + 5 + i).to(torch.float16)
               for i in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")

    def hstep():
        fa.fa_fwd(q, k, v, softmax_scale=w.scale, causal=True, out=o, lse=lse)

    _, per = time_launches(torch, hstep, steps, 10)
    out["fp16_forward"] = launch_stats(w.name + " fp16", fwd_flops(w.B, w.H, w.N, w.D, True), per)
    del q, k, v, o, lse
    wb = ai.BACKWARD
    log("dropout p=0.1:", wb.name)
    q, k, v, do = (gpu_randn_bf16(torch, (wb.B, wb.H, wb.N, wb.D), wb.seed * 10 + 5 + i)
                   for i in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((wb.B, wb.H, wb.N), dtype=torch.float32, device="cuda")
    drop = dict(dropout_p=0.1, seed=1234, offset=0)

    def dfstep():
        fa.fa_fwd(q, k, v, softmax_scale=wb.scale, causal=True, out=o, lse=lse, **drop)

    _, per = time_launches(torch, dfstep, steps, 10)
    fflops = fwd_flops(wb.B, wb.H, wb.N, wb.D, True)
    out["dropout_forward"] = launch_stats(wb.name.replace("bwd", "fwd") + " dropout 0.1", fflops,
                                          per)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_size(wb.B, wb.H, wb.N, wb.D), dtype=torch.uint8,
                     device="cuda")

    def dbstep():
        fa.fa_bwd(q, k, v, o, lse, do, softmax_scale=wb.scale, causal=True, dq=dq, dk=dk,
                  dv=dv, workspace=ws, **drop)

    _, per = time_launches(torch, dbstep, steps, 5)
    out["dropout_backward"] = launch_stats(wb.name + " dropout 0.1", 2.5 * fflops, per)
    del q, k, v, do, o, lse, dq, dk, dv, ws
    return out


def launch_stats(name, flops, per):
    """Per-launch median / min / mean of HIP-event durations (ms) and the
    TFLOP/s of the median against the bf16 peak."""
    med = statistics.median(per)
    return {"workload": name, "launches": len(per), "ms_median": round(med, 4),
            "ms_min": round(min(per), 4), "ms_mean": round(statistics.mean(per), 4),
            "tflops": round(flops / (med * 1e-3) / 1e12, 1),
            "frac": round(flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def run_cold_l2(torch, fwd_step, flops, steps):
    """The metric workload with L2/MALL flushed before each launch: a
    512 MiB scratch write runs between launches and only the attention
    launch is timed."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    per = []
    for i in range(steps + 1):
        scratch.fill_(i & 0xFF)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fwd_step()
        e.record()
        torch.cuda.synchronize()
        if i > 0:
            per.append(s.elapsed_time(e))
    del scratch
    return launch_stats("causal fwd B4 H32 N4096 D128, L2/MALL flushed before each launch",
                        flops, per)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--bwd-steps", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--config-steps", type=int, default=10,
                    help="launches of the varlen, long, chunked-prefill, fp16 and "
                         "dropout workloads and of the flushed-cache run (0 = skip)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device-to-device copy of MIB MiB "
                         "three times (reference for HBM byte counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(heads would shard across GPUs with no exchange); run --gpus 1",
              file=sys.stderr)
        return 2
    rank = int(os.environ.get("RANK", "0"))

    import torch
    import attn_inputs as ai
    import exact_io_aware_44_amd as fa
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    fa.load()

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        log("copy calibration: %d bytes per copy" % nbytes)
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- inputs of the metric, then the other workloads, then the metric ----
    # The GPU's clocks ramp up over roughly 30 ms of work after an idle
    # period (preparing inputs on the host, the oracle run): right after idle
    # the forward's launches take 0.61-0.65 ms, in steady state 0.51-0.52 ms.
    # So the metric's inputs are made first, the other workloads run next,
    # and the metric's warm-up and timed launches follow them directly, on a
    # GPU that has been working for about a second.
    w = ai.CAUSAL
    log("inputs", w.name)
    q, k, v = (x.cuda() for x in ai.qkv(w.B, w.H, w.N, w.D, w.seed))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    # ---- backward against the same roofline, decoding, varlen, long ---------
    t_other = time.perf_counter()
    backward = None
    if args.bwd_steps > 0:
        backward = run_backward(torch, ai, fa, args.bwd_steps)
    decode = None
    if args.decode_steps > 0:
        decode = run_decode(torch, ai, fa, args.decode_steps)
    nexts = run_next_rows(torch, ai, fa, args.config_steps) if args.config_steps > 0 else {}
    others = run_other_configs(torch, ai, fa, args.config_steps) if args.config_steps > 0 else {}
    torch.cuda.synchronize()
    before_s = time.perf_counter() - t_other

    # ---- forward: the metric -------------------------------------------------
    def fwd_step():
        fa.fa_fwd(q, k, v, softmax_scale=w.scale, causal=True, out=o, lse=lse)

    log("forward: %d warmup, %d timed" % (args.warmup, args.steps))
    total_ms, per = time_launches(torch, fwd_step, args.steps, args.warmup)
    flops = fwd_flops(w.B, w.H, w.N, w.D, True)
    ms_per_step = total_ms / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    launch_ms = statistics.mean(per)
    achieved = flops / (launch_ms * 1e-3) / 1e12
    forward_launches = launch_stats(w.name, flops, per)
    forward_launches["other_workloads_before_s"] = round(before_s, 3)
    cold = run_cold_l2(torch, fwd_step, flops, args.config_steps) if args.config_steps > 0 else None
    del q, k, v, o, lse

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": w.name, "batch": w.B, "heads": w.H,
                   "seq_len": w.N, "head_dim": w.D, "causal": True,
                   "flops_per_step": flops,
                   "flop_convention": "4*D per (query,key) pair; causal = half of B*H*N^2"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "fwd_kernel<128, causal>",
                     "avg_launch_ms": round(launch_ms, 5)},
        "forward_launches": forward_launches,
        "forward_cold_l2": cold,
        "backward": backward,
        "decode": decode,
        "varlen": others.get("varlen"),
        "varlen_backward": others.get("varlen_backward"),
        "long": others.get("long"),
        "chunked_prefill": nexts.get("chunked_prefill"),
        "fp16_forward": nexts.get("fp16_forward"),
        "dropout_forward": nexts.get("dropout_forward"),
        "dropout_backward": nexts.get("dropout_backward"),
    }
    if rank == 0 and args.cpu_budget > 0:
        log("cpu baseline (oracle), about %.0f s" % args.cpu_budget)
        line["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    if rank == 0:
        print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
