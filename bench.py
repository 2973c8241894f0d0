#!/usr/bin/env python3
"""Benchmark: verified draft positions per second on one MI355X.

A step is one verify round of the whole path on one batch of synthetic input:
confidence truncation (when the workload truncates), LM-head logits with row
statistics, then greedy or rejection-sampling acceptance with the correction
or bonus token. Inputs are staged in HBM before timing; the timed steps run
as one HIP-graph replay. Verified positions are counted on the GPU (the
drafts-verified counter, sum over requests of L_r).

Default workload: high-concurrency rejection verify, B=128 requests with
gamma=16 drafts each, d=7168, V=129280, T=1.0, confidence-truncated ragged
lengths (about 956 verified rows per step), 8 distinct seeded steps staged
in HBM and cycled. The LM-head contraction is a dense bf16 MFMA problem here
(about 1.8 TFLOP per step). Smaller LM heads (--workload greedy-block9, 134
MB) would stay resident in the 256 MB last-level cache between steps, so
copies are rotated until every step streams its head from HBM.

Prints one JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--preheat-seconds", type=float, default=1.0,
                    help="before the first timed region, run untimed steps for this long, so "
                         "that the timed steps see the clocks the GPU sustains under this load "
                         "(0 = none)")
    ap.add_argument("--workload", default="concurrency-b128",
                    help="tiny-greedy, greedy-block9, rejection-b1, ragged-b32 or "
                         "concurrency-b128 (default)")
    ap.add_argument("--distinct", type=int, default=None,
                    help="distinct pre-staged steps cycled through (default: all for the "
                         "greedy block workload, 8 otherwise)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU-oracle baseline sample (0 = skip)")
    ap.add_argument("--eager", action="store_true", help="launch steps eagerly, no HIP graph")
    ap.add_argument("--kernel-only", action="store_true",
                    help="time only the LM-head contraction kernel (for profiler runs)")
    ap.add_argument("--accept-rate", action="store_true",
                    help="rejection workloads: also compute the analytic acceptance rate of "
                         "every verified position (sd_accept_rejection_ex)")
    ap.add_argument("--scheduler", choices=["threshold", "early-stop", "top-k"],
                    default="threshold",
                    help="truncating workloads: confidence threshold (default) or the "
                         "hardware-aware prefix scheduler on an SPS table profiled at start "
                         "(top-k sizes the batch from the confidences of two steps before)")
    ap.add_argument("--weights", choices=["auto", "bf16", "w12", "blocked"], default="auto",
                    help="LM-head format: bf16 [V][d]; the lossless W12 stream (encoded on the "
                         "host before timing); or the same bf16 weights re-laid in 64x128 slab "
                         "blocks (sd_lm_head_block, before timing). w12 and blocked: streaming "
                         "regime only. auto (default): blocked in the streaming regime "
                         "(B (gamma + 1) <= 64, d % 128 == 0), else bf16")
    ap.add_argument("--decode-loop", action="store_true",
                    help="instead of the verify benchmark: the toy multi-step decode loop "
                         "(bigram target over the workload's LM head, drafter table right 75%% "
                         "of the time) replayed from a HIP graph; reports emitted tokens/s")
    ap.add_argument("--step-times-from-trace", metavar="KERNEL_TRACE_CSV", default=None,
                    help="no GPU run: read a rocprofv3 kernel trace of a bench.py run and print "
                         "the median and p10/p90 of the per-step times of its first timed region")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before timing, run one device-to-device copy of this many MiB "
                         "(the known-size reference for the profiler's HBM byte counters)")
    return ap.parse_args()


def contraction_kernel(w) -> str:
    """Name of the kernel sd_verify_contraction launches for this shape."""
    cap = w.B * (w.gamma + 1)
    if cap <= 64:
        return "k_gemm_skinny" if w.d % 128 == 0 else "k_gemm_stream"
    return "k_gemm_dma" if w.d % 64 == 0 else "k_gemm_tile"


def kernel_source_hash() -> str:
    """Hash of the sources the contraction kernels are compiled from."""
    h = hashlib.sha256()
    for f in ["sd_gemm.hip", "sd_internal.h"]:
        with open(os.path.join(ROOT, "draft_block_verification_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def step_times_from_trace(path):
    """Per-step times of the first timed region in a rocprofv3 kernel trace of bench.py.

    The timed region lies between the first two marker kernels (torch's spin kernel).
    A step starts with the first kernel of the path (truncation or scheduling when the
    workload truncates, else the contraction); a step's time runs from its first
    kernel's start to the next step's, and for the last step to its last kernel's end.
    """
    import csv
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    marks = [i for i, r in enumerate(rows) if "spin" in r["Kernel_Name"].lower()]
    if len(marks) < 2:
        sys.exit("no pair of marker kernels in the trace")
    region = rows[marks[0] + 1:marks[1]]
    names = [r["Kernel_Name"] for r in region]
    first = next((k for k in ("k_truncate", "k_schedule") if any(k in n for n in names)), "k_gemm")
    starts = [i for i, n in enumerate(names) if first in n]
    t = [int(region[i]["Start_Timestamp"]) for i in starts]
    t.append(max(int(r["End_Timestamp"]) for r in region))
    per = np.diff(np.array(t, dtype=np.float64)) / 1e3
    out = {"steps": len(per), "first_kernel": first, "median_us": float(np.median(per)),
           "p10_us": float(np.percentile(per, 10)), "p90_us": float(np.percentile(per, 90)),
           "mean_us": float(per.mean())}
    print(json.dumps(out))


def main():
    args = parse()
    if args.step_times_from_trace:
        return step_times_from_trace(args.step_times_from_trace)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the verify path "
              "runs on one GPU, which holds the whole LM head.", file=sys.stderr)
        sys.exit(2)

    import torch
    import draft_block_verification_amd as sd
    from synth import make_step, make_weights, workload

    w = workload(args.workload)
    if args.decode_loop:
        return decode_loop_bench(args, w)
    K = args.steps if args.steps is not None else (1000 if w.name == "greedy-block9" else 50)
    Wu = args.warmup
    S = args.distinct or (w.steps if w.name in ("greedy-block9", "tiny-greedy") else 8)
    S = max(1, min(S, w.steps))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    if args.weights == "auto":
        # The blocked copy is a one-time re-layout of static weights that the streaming
        # contraction reads as contiguous stages; the tiled regime reads [V][d].
        streaming = w.B * (w.gamma + 1) <= 64 and w.d % 128 == 0
        args.weights = "blocked" if streaming else "bf16"

    # ---- stage inputs in HBM
    W = make_weights(w)
    if args.weights == "w12":
        enc = sd.w12_encode(W)
        w_bytes = enc[0].nbytes + enc[1].nbytes
        make_head = lambda: sd.W12Weights(*enc, device=dev)
    elif args.weights == "blocked":
        w_bytes = W.nbytes                      # the same bf16 weights, re-laid in slab blocks
        make_head = lambda: sd.BlockedWeights(bf16_dev(W))
    else:
        w_bytes = W.nbytes
        make_head = lambda: bf16_dev(W)
    n_copies = max(1, math.ceil(2 * MALL_BYTES / w_bytes)) if w_bytes < MALL_BYTES else 1
    W_dev = [make_head() for _ in range(n_copies)]
    steps_host = [make_step(w, W, i) for i in range(S)]
    def conditional(conf):
        """Per-position conditional confidences c_k = s_k / s_(k-1) of survival curves s."""
        c = conf.astype(np.float32).copy()
        c[:, 1:] = conf[:, 1:] / conf[:, :-1]
        return c

    staged = []
    for s in steps_host:
        staged.append(dict(
            hidden=bf16_dev(s.hidden),
            draft_tokens=torch.from_numpy(s.draft_tokens).to(dev),
            conf=None if s.conf is None else torch.from_numpy(s.conf).to(dev),
            cond=None if s.conf is None else torch.from_numpy(conditional(s.conf)).to(dev),
            draft_logits=None if s.draft_logits is None else bf16_dev(s.draft_logits),
            u_accept=torch.from_numpy(s.u_accept).to(dev),
            u_resample=torch.from_numpy(s.u_resample).to(dev)))
    sched = None
    sps = None
    if args.scheduler != "threshold":
        if not w.truncate:
            sys.exit(f"--scheduler needs a truncating workload; {w.name} verifies whole blocks")
        sched = sd.SCHED_EARLY_STOP if args.scheduler == "early-stop" else sd.SCHED_TOP_K
        sps = sd.profile_sps(w.B, w.gamma, W_dev[0], w.T)
    vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold, device=dev,
                        accept_rate=args.accept_rate, scheduler=sched, sps=sps)
    stream = torch.cuda.Stream(device=dev)

    # The threshold reads survival confidences; the scheduler reads the conditional ones
    # (its own running product rebuilds the survival).
    conf_key = "conf" if sched is None else "cond"

    def step(i):
        st = staged[i % S]
        stale = staged[(i - 2) % S]["cond"] if sched == sd.SCHED_TOP_K else None
        vr.run(st["hidden"], W_dev[i % n_copies], st["draft_tokens"], st[conf_key],
               st["draft_logits"], st["u_accept"], st["u_resample"], conf_stale=stale)

    def verify_only(i):
        # The contraction kernel alone: the same launch sd_verify_logits starts with.
        st = staged[i % S]
        sd.sd_verify_contraction(st["hidden"], W_dev[i % n_copies], vr.verify_len,
                                 vr.row_offsets, w.T, vr.logits, vr.ws_verify)

    preheated = [args.preheat_seconds <= 0]

    def timed(fn, n, warm):
        """Run fn(i) for n steps after `warm` untimed ones; returns milliseconds. Before the
        first timed region, untimed steps run for --preheat-seconds (the clocks ramp over
        the first tens of milliseconds of sustained load)."""
        if not preheated[0]:
            t_end = time.time() + args.preheat_seconds
            i = 0
            while time.time() < t_end:
                with torch.cuda.stream(stream):
                    for _ in range(8):
                        fn(i)
                        i += 1
                torch.cuda.synchronize()
            preheated[0] = True
        with torch.cuda.stream(stream):
            for i in range(warm):
                fn(i)
        torch.cuda.synchronize()
        graph = None
        if not args.eager:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(n):
                    fn(warm + i)
            torch.cuda.synchronize()
        vr.counters.zero_()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            # Marker kernels outside the events bracket the timed steps in a kernel
            # trace (see --step-times-from-trace).
            torch.cuda._sleep(1000)
            e0.record(stream)
            if graph is not None:
                graph.replay()
            else:
                for i in range(n):
                    fn(warm + i)
            e1.record(stream)
            torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- whole-path timing
    if args.kernel_only:
        ms_total = timed(verify_only, K, Wu)
        positions = None
    else:
        ms_total = timed(step, K, Wu)
        positions = int(vr.counters[0].item())
    # Rows per step from the same staged inputs (a truncation pass per distinct step).
    def rows_of(i):
        """(rows, expected tokens) of step i: tau = R + sum of the admitted survivals."""
        st = staged[i % S]
        if not w.truncate:
            return w.B * (w.gamma + 1), None
        if sched is None:
            vl, _ = sd.sd_truncate_by_confidence(st["conf"], w.threshold)
        else:
            stale = staged[(i - 2) % S]["cond"] if sched == sd.SCHED_TOP_K else None
            vl, _ = sd.sd_schedule_prefix(st["cond"], sps, sched, stale)
        vl = vl.cpu().numpy()
        surv = steps_host[i % S].conf
        tau = w.B + float(sum(surv[r, :vl[r]].astype(np.float64).sum() for r in range(w.B)))
        return int(vl.sum()) + w.B, tau

    by_phase = [rows_of(i) for i in range(S)]      # rows depend on the step only through i % S
    mean_rows = float(np.mean([by_phase[i % S][0] for i in range(Wu, Wu + K)]))
    tau = (float(np.mean([by_phase[i % S][1] for i in range(Wu, Wu + K)])) if w.truncate
           else None)
    torch.cuda.synchronize()
    if positions is None:
        positions = int(round((mean_rows - w.B) * K))

    # ---- dominant kernel: the LM-head contraction, timed alone (graph of K launches).
    # It runs on the row layout the last step left in place (truncation included).
    rows_c = int(vr.row_offsets[-1].item()) if w.truncate else w.B * (w.gamma + 1)
    ms_verify = timed(verify_only, K, Wu) / K
    # Algorithmic bytes: the LM head once (in its stored format) plus the verified hidden rows.
    v_bytes = w_bytes + rows_c * w.d * 2
    v_flops = 2.0 * rows_c * w.V * w.d
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if v_flops / v_bytes > ridge:
        roof = {"bound": "mfma", "achieved": v_flops / (ms_verify * 1e-3) / 1e12,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": v_bytes / (ms_verify * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    tr_path = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tr_path):
        tr = json.load(open(tr_path))
        ent = tr.get(w.name if args.weights == "bf16" else f"{w.name}-{args.weights}")
        if ent and ent.get("kernel_hash") == kernel_source_hash():
            roof["traffic"] = ent["bytes_per_launch"]
    roof["kernel"] = contraction_kernel(w)
    roof["avg_launch_us"] = ms_verify * 1e3
    roof["rows"] = rows_c

    ms_step = ms_total / K
    value = positions / (ms_total * 1e-3)
    # The whole step against its own roofline: algorithmic bytes (LM head once, verified
    # hidden rows, kept drafter rows when T > 0) and flops (2 M V d) of an average timed
    # step; its roofline time is the larger of bytes / HBM peak and flops / MFMA peak.
    mean_pos = mean_rows - w.B
    s_bytes = w_bytes + mean_rows * w.d * 2 + (mean_pos * w.V * 2 if w.T > 0 else 0.0)
    s_flops = 2.0 * mean_rows * w.V * w.d
    t_roof = max(s_bytes / (HBM_PEAK_GBS * 1e9), s_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    roof["step_bound"] = ("mfma" if s_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) >=
                          s_bytes / (HBM_PEAK_GBS * 1e9) else "hbm")
    roof["step_roofline_us"] = t_roof * 1e6
    roof["step_frac"] = t_roof / (ms_step * 1e-3)
    roof["roofline_positions_per_s"] = mean_pos / t_roof

    # ---- CPU oracle baseline on a bounded sample of the same steps
    cpu = None
    if args.cpu_seconds > 0:
        from threadpoolctl import threadpool_info, threadpool_limits
        from oracle import sd_oracle as O
        host_cores = len(os.sched_getaffinity(0))
        W64 = O.lm_head_f64(W)
        done_pos, t_cpu, n_cpu = 0, 0.0, 0
        # The oracle's matmul is the only multi-threaded part; let its BLAS use every
        # core this process may run on.
        with threadpool_limits(limits=host_cores, user_api="blas"):
            blas = [p.get("num_threads", 1) for p in threadpool_info()
                    if p.get("user_api") == "blas"]
            while t_cpu < args.cpu_seconds and n_cpu < 10 * S:
                s = steps_host[n_cpu % S]
                t0 = time.perf_counter()
                res = O.verify_step(s.hidden, W64, s.draft_tokens, w.T,
                                    conf=s.conf if w.truncate else None, threshold=w.threshold,
                                    draft_logit_bits=s.draft_logits, u_accept=s.u_accept,
                                    u_resample=s.u_resample)
                t_cpu += time.perf_counter() - t0
                done_pos += int(res.accept.counters[0])
                n_cpu += 1
        del W64
        cpu = {"value": done_pos / t_cpu, "unit": "verified draft positions/s",
               "cores": int(max(blas) if blas else 1), "host_cores": host_cores,
               "kind": "oracle",
               "sample": f"{n_cpu} whole steps of {w.name} ({done_pos} verified positions, "
                         f"{t_cpu:.1f} s; fp64 numpy oracle, inputs pre-generated)"}

    out = {
        "metric": "verified draft positions/sec at 1 GPU; % HBM or MFMA roofline",
        "value": value,
        "unit": "verified draft positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "preheat_s": args.preheat_seconds,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "gamma": w.gamma, "d": w.d, "V": w.V,
                   "temperature": w.T, "truncate": w.truncate, "distinct_steps": S,
                   "lm_head_copies": n_copies, "mean_rows": mean_rows,
                   "launch": "eager" if args.eager else "hipgraph",
                   "accept_rate": vr.accept_rate is not None,
                   "scheduler": args.scheduler,
                   "lm_head_format": args.weights,
                   # Expected tokens per second if the confidences are calibrated survival
                   # probabilities: (R + admitted survivals) per step / step time.
                   "expected_tokens_per_s": None if tau is None else tau / (ms_step * 1e-3),
                   "timed": "verify only" if args.kernel_only else "truncate+verify+accept"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def decode_loop_bench(args, w):
    """Toy decode loop: greedy speculative decoding of a bigram target whose hidden state
    is an embedding row planted toward a successor token's LM-head row; the drafter
    proposes the target's choice 75% of the time. Steps are captured three at a time in a
    HIP graph; the timed region replays it."""
    import torch
    import draft_block_verification_amd as sd
    from draft_block_verification_amd.decode_loop import ToyDecodeLoop
    from synth import make_weights

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W = make_weights(w)
    Wd = torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).to(dev).view(torch.bfloat16)
    gen = torch.Generator(device="cpu").manual_seed(7)
    succ = torch.randperm(w.V, generator=gen).to(dev)
    Wf = Wd[succ].float()
    E = (0.3 * torch.randn((w.V, w.d), generator=gen).to(dev) / w.d ** 0.5 +
         4.0 * Wf / Wf.norm(dim=1, keepdim=True)).to(torch.bfloat16)
    del Wf
    nxt = torch.empty(w.V, dtype=torch.int64, device=dev)
    for v0 in range(0, w.V, 4096):                    # the target's greedy next token
        nxt[v0:v0 + 4096] = (E[v0:v0 + 4096].float() @ Wd.float().T).argmax(1)
    right = torch.rand(w.V, generator=gen).to(dev) < 0.75
    dnext = torch.where(right, nxt, torch.randint(0, w.V, (w.V,), generator=gen).to(dev))
    dconf = torch.where(right, torch.full((w.V,), 0.92, device=dev),
                        0.2 + 0.4 * torch.rand(w.V, generator=gen).to(dev))
    B, g = max(w.B, 8), w.gamma
    reps = max(1, (args.steps or 300) // 3)
    loop = ToyDecodeLoop(Wd, E, dnext, dconf, B, g, 3 * (reps + 1))
    start = torch.randint(0, w.V, (B,), generator=gen).to(dev)
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        loop.reset(start)
        for i in range(3):
            loop.step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for i in range(3):
            loop.step(i)
    with torch.cuda.stream(s):
        loop.reset(start)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(reps):
            graph.replay()
        e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    emitted = int((loop.length - 1).sum().item())
    drafted, accepted = loop.vr.counters.cpu().tolist()
    out = {"metric": "toy decode loop emitted tokens/s (greedy speculative decoding, 1 GPU)",
           "value": emitted / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": 3 * reps,
           "ms_per_step": ms / (3 * reps), "higher_is_better": True, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": f"decode-loop-{w.name}", "B": B, "gamma": g, "d": w.d, "V": w.V,
                      "drafted": drafted, "accepted": accepted,
                      "tokens_per_request_step": emitted / (3 * reps * B),
                      "launch": "hipgraph (3 steps per graph)"}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
