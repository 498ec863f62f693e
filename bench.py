#!/usr/bin/env python3
"""Benchmark one batched verification step on one MI355X.

Workload: B=64 requests, K=4 drafts, V=128256, bf16 logits (target ~ N(0, 3^2)
plus a +6 spike per row, draft = target + N(0, 0.7^2)), T = 1, no filters,
seeded synthetic inputs.  A "step" is one full call: row statistics, accept
scan and the float64 residual / bonus draw for every request.

Output: exactly one JSON line on stdout (progress goes to stderr):
  value            verified draft positions per second (sum of draft lengths / step time)
  ms_per_step      mean step time over the timed region (HIP events on the call's stream)
  host_us_per_call host time to enqueue one call from Python (below ms_per_step: the
                   timed steps are GPU-bound, not launch-bound)
  roofline         the dominant kernel (row statistics): algorithmic bytes per launch
                   over its mean duration (a burst of launches between two HIP events),
                   against the 8 TB/s HBM peak
  us_per_call      median, p10 and p90 of single calls (a pass with one event per call)
  cpu_baseline     the fp64 oracle on this host, on a bounded sample of the same workload
Inputs rotate over several independent sets whose total exceeds twice the
256 MB last-level cache, so reads come from HBM.

--workload N runs the same measurement on the other synthetic workloads (1: B=8,
K=4, V=4096 fp32; 2: B=1, K=5, V=32000 bf16, T=0.8; 4: B=256, K=8, V=152064 fp32,
T=0.7, top-k 50 then top-p 0.9; 5: B=64, ragged drafts up to 8, V=129280 bf16,
EOS), for reference next to the headline.  On workload 4 the draft tokens are
drawn from the processed draft rows by the library's own sampler (specv_sample),
and the dominant kernel is the top-k candidate pass, timed per call.
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# HBM bytes of one launch of each workload's dominant kernel, from rocprofv3
# FETCH_SIZE and WRITE_SIZE runs scaled by a plain-copy calibration (see the
# profiles directory), each valid only for the sources it was measured on:
# the row-statistics pass of the headline workload, the top-k candidate pass
# of B=256, K=8, V=152064 fp32 (top-k 50, top-p 0.9) and the radix select of
# the headline shape with top-p 0.9 alone.
TRAFFIC = {
    "B64_K4_V128256_bf16": {
        "sources": ("row_stats.hip", "row_core.h", "common.h"),
        "sources_sha256_16": "a9a4a3778ecb2f8c", "bytes": 148143669},
    "B256_K8_V152064_f32_topk50_topp0.9": {
        "sources": ("filter.hip", "filter_common.h", "radix_select.h", "wave_scan.h", "exp64.h",
                    "common.h"),
        "sources_sha256_16": "6169525b906dbe31", "bytes": 2687319207},
    "B64_K4_V128256_bf16_topp0.9": {
        "sources": ("filter_rows.hip", "filter_common.h", "hist_select.h", "radix_select.h",
                    "wave_scan.h", "exp64.h", "common.h"),
        "sources_sha256_16": "c5def2af1ca982a7", "bytes": 148253874},
}
# The same for one LM-head launch at M=320, D=4096, V=128256 (scaled by the
# copy calibration taken with the row-statistics figure).
LM_HEAD_TRAFFIC = {"sources": ("lm_head.hip", "common.h"),
                   "sources_sha256_16": "42a7e1a86d6396e3", "bytes": 1180264466}


def measured_traffic(entry):
    """An entry's bytes while its sources are the measured ones, else None."""
    if entry is None or entry["bytes"] is None:
        return None
    return entry["bytes"] if sources_hash(entry["sources"]) == entry["sources_sha256_16"] else None


WORKLOAD = 3
METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak) at B=64,K=4,V=128k"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw HIP events (the call records them on its own stream)."""

    def __init__(self, n):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = h

    def elapsed_ms(self, i, j):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for h in self.arr:
            self.lib.hipEventDestroy(h)


def sources_hash(files=("row_stats.hip", "common.h")):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "speculative_decoding_sampling_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where it is absent)."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_groups(B, group):
    return ([list(range(B))] if group is None else
            [list(range(i, min(i + group, B))) for i in range(0, B, group)])


def _time_oracle(w, groups, budget_s):
    """Verify ``groups`` of requests of ``w`` in turn with the oracle until
    ``budget_s`` seconds of oracle time; returns (positions, seconds, calls)."""
    import oracle as O
    reps, t_total, positions = 0, 0.0, 0
    while t_total < budget_s:
        reqs = groups[reps % len(groups)]
        t0 = time.perf_counter()
        O.verify(w.target, w.draft, w.draft_tokens, w.draft_len, w.u, w.u_final, w.T, w.top_k,
                 w.top_p, w.eos_id, w.dtype, requests=reqs)
        t_total += time.perf_counter() - t0
        positions += int(np.sum(w.draft_len[reqs]))
        reps += 1
    return positions, t_total, reps


def _oracle_worker(job):
    """One process of the all-cores leg: rebuild the workload from its seed
    (the drafted tokens are passed in when they came from the GPU sampler),
    then time the oracle on this worker's share of the requests."""
    wl, seed, tokens, groups, budget_s = job
    from speculative_decoding_sampling_amd.workloads import make_workload
    w = make_workload(wl, seed=seed,
                      draft_sampler=(lambda z, T, k, p, x: 0) if tokens is not None else None)
    if tokens is not None:
        w.draft_tokens = tokens
    t0 = time.perf_counter()
    pos, secs, calls = _time_oracle(w, groups, budget_s)
    return pos, secs, calls, time.perf_counter() - t0


def cpu_baseline(w, budget_s, group=None, tokens_from_gpu=False):
    """Time the fp64 oracle on the same workload on this host's cores.

    Single core: whole calls (or groups of ``group`` requests in turn where a
    whole call is too long for the budget), pinned to one core.  All cores:
    one spawned process per core (at most 16), each rebuilding the workload
    from its seed and timing the oracle on its own share of the requests for
    the same budget; the rate is all their positions over the longest
    worker's timed span.  The all-cores figure is the reported value."""
    groups = _oracle_groups(w.B, group)
    allowed = os.sched_getaffinity(0)
    try:
        os.sched_setaffinity(0, {min(allowed)})
        pos1, t1, reps1 = _time_oracle(w, groups, budget_s)
    finally:
        os.sched_setaffinity(0, allowed)
    if group is None:
        what = f"whole calls of the same workload (B={w.B}, K={w.K}, V={w.V})"
    else:
        what = f"groups of {group} requests of the same workload (B={w.B}, K={w.K}, V={w.V})"
    single = {"value": pos1 / t1, "cores": 1,
              "sample": f"{reps1} {what}, {t1:.1f} s of numpy fp64 pinned to one core",
              "seconds_per_call": t1 / reps1 * (1 if group is None else w.B / group)}

    ncores = max(1, min(16, len(allowed)))
    import multiprocessing as mp
    share = [[b for b in range(w.B) if b % ncores == i] for i in range(ncores)]
    jobs = []
    for i in range(ncores):
        if not share[i]:
            continue
        sub = ([share[i]] if group is None else
               [share[i][j:j + group] for j in range(0, len(share[i]), group)])
        jobs.append((w.cfg, w.seed, w.draft_tokens if tokens_from_gpu else None, sub, budget_s))
    with mp.get_context("spawn").Pool(len(jobs)) as pool:
        res = pool.map(_oracle_worker, jobs)
    pos_all = sum(r[0] for r in res)
    span = max(r[3] for r in res)
    calls = sum(r[2] for r in res)
    return {"value": pos_all / span, "unit": "positions/s", "cores": len(jobs), "kind": "oracle",
            "sample": (f"{len(jobs)} processes, each verifying its share of the requests of the "
                       f"same workload (B={w.B}, K={w.K}, V={w.V}) for {budget_s:.0f} s of numpy "
                       f"fp64 ({calls} oracle calls in all, {span:.1f} s wall)"),
            "single_core": single, "cpu_model": cpu_model()}


def bench_sample(args):
    """The draft model's sampling step on the headline workload: one draw from
    the processed distribution of each of the 256 draft rows (B=64 x K=4,
    V=128256, bf16, T=1), through specv_sample."""
    import torch
    from speculative_decoding_sampling_amd import binding
    from speculative_decoding_sampling_amd.build import LIB
    from speculative_decoding_sampling_amd.workloads import WORKLOADS, make_workload, uniforms

    if not os.path.exists(LIB):
        from speculative_decoding_sampling_amd.build import build
        build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets = []
    for i in range(args.sets):
        w = make_workload(WORKLOAD, seed=1000 + WORKLOAD + 100 * i)
        rows = np.ascontiguousarray(w.draft.reshape(-1, w.V))
        u = uniforms(np.random.default_rng(5000 + i), rows.shape[0])
        sets.append(dict(
            logits=torch.from_numpy(rows.view(np.int16)).to(dev).view(torch.bfloat16),
            u=torch.from_numpy(u).to(dev),
            out=torch.empty(rows.shape[0], dtype=torch.int32, device=dev)))
    R, V, T = rows.shape[0], w.V, w.T
    alg_bytes = R * V * 2
    stream = torch.cuda.current_stream(dev)
    ws = torch.empty(binding.workspace_bytes(R, 0, V, torch.bfloat16), dtype=torch.uint8,
                     device=dev)

    def step(i):
        st = sets[i % len(sets)]
        binding.sample(st["logits"], st["u"], T, out_tokens=st["out"], workspace=ws,
                       stream=stream)

    for i in range(args.warmup):
        step(i)
    ev = HipEvents(2)
    torch.cuda.synchronize()
    ev.lib.hipEventRecord(ev.arr[0], stream.cuda_stream)
    for i in range(args.steps):
        step(i)
    ev.lib.hipEventRecord(ev.arr[1], stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / args.steps
    ev.close()
    y = sets[0]["out"].cpu().numpy()
    assert np.all((y >= 0) & (y < V)), y
    log(f"sample: {ms * 1e3:.2f} us/step for {R} rows")
    print(json.dumps({
        "metric": "draft tokens drawn/sec (processed-distribution sampler)", "value": R / (ms * 1e-3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32+f64", "data": "synthetic",
        "config": {"workload": WORKLOADS[WORKLOAD]["name"] + " draft rows", "rows": R, "V": V,
                   "logits": "bf16", "temperature": T, "top_k": 0, "top_p": 1.0,
                   "algorithmic_bytes_per_step": alg_bytes},
        "hbm_gbps_whole_step": alg_bytes / (ms * 1e-3) / 1e9}), flush=True)


def bench_rates(args):
    """Acceptance diagnostics on the headline workload (B=64, K=4, V=128256,
    bf16, T=1): specv_acceptance_rates (the row statistics, then a second
    pass over each drafted row pair for sum_x min(p(x), q(x))), and on one
    verified round's outcome specv_round_stats and the device-resident
    DraftLengthMonitor update.  Reported for reference next to the headline."""
    import torch
    from speculative_decoding_sampling_amd import binding
    from speculative_decoding_sampling_amd.build import LIB
    from speculative_decoding_sampling_amd.workloads import WORKLOADS, make_workload, upload

    if not os.path.exists(LIB):
        from speculative_decoding_sampling_amd.build import build
        build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets, hosts = [], []
    for i in range(args.sets):
        w = make_workload(WORKLOAD, seed=1000 + WORKLOAD + 100 * i)
        hosts.append(w)
        a = upload(w, dev)
        a["beta"] = torch.empty((w.B, w.K), dtype=torch.float32, device=dev)
        sets.append(a)
    w0 = hosts[0]
    B, K, V = w0.B, w0.K, w0.V
    positions = w0.positions
    # two reads of each drafted (target, draft) row pair: one for the row
    # statistics, one for the sums of min(p, q)
    drafted = int(np.sum(w0.draft_len))
    alg_bytes = 2 * (2 * drafted * V * 2)
    stream = torch.cuda.current_stream(dev)
    ws = torch.empty(binding.workspace_bytes(B, K, V, torch.bfloat16), dtype=torch.uint8,
                     device=dev)

    def rates(i):
        st = sets[i % len(sets)]
        binding.acceptance_rates(st["target_logits"], st["draft_logits"], st["draft_len"], w0.T,
                                 beta=st["beta"], workspace=ws, stream=stream)

    ev = HipEvents(args.steps + 1)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev.lib.hipEventRecord(ev.arr[i], stream.cuda_stream)
            fn(i)
        ev.lib.hipEventRecord(ev.arr[args.steps], stream.cuda_stream)
        torch.cuda.synchronize()
        us = np.array([ev.elapsed_ms(i, i + 1) for i in range(args.steps)]) * 1e3
        return float(ev.elapsed_ms(0, args.steps) / args.steps * 1e3), us

    rates_us, rates_calls = timed(rates)
    b = sets[0]["beta"].cpu().numpy()
    assert np.all((b > 0) & (b <= 1)), "every position is drafted in this workload"
    # one verified round per set, then its statistics and the monitor update
    outs = []
    for st in sets:
        r = binding.verify(**{k: v for k, v in st.items() if k != "beta"}, workspace=ws,
                           stream=stream)
        outs.append((st, r["out_tokens"], r["n_emitted"]))
    mon = binding.DraftLengthMonitor(B, 16, 8, dev, stream=stream)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    rate = torch.empty(B, dtype=torch.float64, device=dev)

    def round_stats(i):
        st, out, n = outs[i % len(outs)]
        binding.round_stats(st["draft_tokens"], st["draft_len"], out, n, st["beta"], stream=stream)

    def monitor(i):
        st, out, n = outs[i % len(outs)]
        mon.update(st["draft_tokens"], st["draft_len"], out, n, next_draft_len=nxt, rate=rate,
                   stream=stream)

    stats_us, _ = timed(round_stats)
    mon_us, _ = timed(monitor)
    ev.close()
    p10, med, p90 = (float(x) for x in np.percentile(rates_calls, [10, 50, 90]))
    gbps = alg_bytes / (rates_us * 1e-6) / 1e9
    log(f"acceptance rates: {rates_us:.2f} us/call (median {med:.2f}), {gbps:.0f} GB/s; "
        f"round stats {stats_us:.2f} us; monitor update {mon_us:.2f} us")
    result = {
        "metric": "per-position acceptance rates sum_x min(p, q): drafted positions/sec",
        "value": positions / (rates_us * 1e-6), "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": rates_us * 1e-3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[WORKLOAD]["name"] + " acceptance rates", "B": B, "K": K,
                   "V": V, "logits": "bf16", "temperature": float(w0.T),
                   "input_sets": args.sets, "positions_per_step": positions,
                   "algorithmic_bytes_per_step": alg_bytes},
        "us_per_call": {"median": med, "p10": p10, "p90": p90},
        "roofline": {"bound": "hbm", "kernel": "row_stats + beta_pass (whole call)",
                     "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None, "launch_us": rates_us,
                     "bytes_per_launch": alg_bytes},
        # both are a few-microsecond kernel behind a Python call: these per-call
        # times are the host's enqueue rate, not the GPU's
        "round_stats_host_bound_us_per_call": stats_us,
        "monitor_update_host_bound_us_per_call": mon_us,
    }
    if not args.no_cpu_baseline:
        import oracle as O
        log(f"timing the oracle for about {args.cpu_seconds:.0f} s")
        t_total, reps = 0.0, 0
        while t_total < args.cpu_seconds:
            t1 = time.perf_counter()
            O.acceptance_rates(w0.target, w0.draft, w0.draft_len, w0.T, dtype=w0.dtype)
            t_total += time.perf_counter() - t1
            reps += 1
        result["cpu_baseline"] = {
            "value": positions * reps / t_total, "unit": "positions/s", "cores": 1,
            "kind": "oracle", "sample": f"{reps} whole calls of the same workload, "
                                        f"{t_total:.1f} s of single-threaded numpy fp64"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def bench_lm_head(args):
    """The verification fused with the target LM head (specv_verify_lm_head)
    at B=64, K=4, V=128256 with a D=4096 LM head: the target logits are
    produced on the matrix cores from synthetic hidden states and weights
    (small-integer values, so the float32 sums are exact) and reduced to row
    statistics in the same kernel.  The weights are repacked once, before
    the timed region, as at model load.  Reported for reference next to the
    headline verification."""
    import torch
    import oracle as O
    from oracle import lm_head as OL
    from speculative_decoding_sampling_amd import binding
    from speculative_decoding_sampling_amd.build import LIB
    from speculative_decoding_sampling_amd.workloads import make_lm_head_workload, upload_lm_head

    if not os.path.exists(LIB):
        from speculative_decoding_sampling_amd.build import build
        build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, K, V, D = 64, 4, 128256, 4096
    t0 = time.perf_counter()
    w = make_lm_head_workload(B, K, V, D, seed=3003)
    log(f"LM-head workload B={B} K={K} V={V} D={D}: {time.perf_counter() - t0:.1f} s to generate")
    a = upload_lm_head(w, dev)
    M = B * (K + 1)
    tl = torch.empty((B, K + 1, V), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    n = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = torch.empty(binding.lm_head_workspace_bytes(B, K, V, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.verify_lm_head(**a, target_logits=tl, out_tokens=out, n_emitted=n, workspace=ws,
                               stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents(2)
    ev.lib.hipEventRecord(ev.arr[0], stream.cuda_stream)
    for _ in range(args.steps):
        step()
    ev.lib.hipEventRecord(ev.arr[1], stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / args.steps
    nn = n.cpu().numpy()
    assert np.all((nn >= 1) & (nn <= w.draft_len + 1)), nn
    # the LM-head kernel alone, for the roofline
    reps = max(10, args.steps // 4)
    logits = tl.view(M, V)
    tws = torch.empty(M * ((V + 255) // 256) * 8, dtype=torch.uint8, device=dev)
    ev.lib.hipEventRecord(ev.arr[0], stream.cuda_stream)
    binding.bench_lm_head(a["hidden"].view(M, D), a["packed_weight"], logits, tws, reps,
                          temperature=w.T, stream=stream, start=ev.arr[0], stop=ev.arr[1])
    torch.cuda.synchronize()
    k_us = ev.elapsed_ms(0, 1) / reps * 1e3
    # context only: the vendor GEMM (torch.matmul, hipBLASLt on ROCm) on the
    # same row-major bf16 operands, logits alone, no statistics
    wt = torch.from_numpy(w.weight.view(np.int16)).to(dev).view(torch.bfloat16)
    ref = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
    hid2 = a["hidden"].view(M, D)
    for _ in range(3):
        torch.matmul(hid2, wt.t(), out=ref)
    torch.cuda.synchronize()
    ev.lib.hipEventRecord(ev.arr[0], stream.cuda_stream)
    for _ in range(reps):
        torch.matmul(hid2, wt.t(), out=ref)
    ev.lib.hipEventRecord(ev.arr[1], stream.cuda_stream)
    torch.cuda.synchronize()
    blas_us = ev.elapsed_ms(0, 1) / reps * 1e3
    del wt, ref
    ev.close()
    flops = 2.0 * M * V * D
    hbm_bytes = V * D * 2 + M * D * 2 + M * V * 2       # weights and hidden read once, logits written
    log(f"lm_head fused step {ms * 1e3:.1f} us; LM-head kernel {k_us:.1f} us "
        f"({flops / k_us / 1e6:.0f} TFLOP/s, {hbm_bytes / k_us / 1e3:.0f} GB/s); "
        f"torch.matmul on the same operands {blas_us:.1f} us")
    result = {
        "metric": "verified draft positions/sec, verification fused with the target LM head",
        "value": w.positions / (ms * 1e-3), "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 MFMA (fp32 accumulate) + f32/f64 verification", "data": "synthetic",
        "config": {"workload": f"B{B}_K{K}_V{V}_D{D}_lm_head_bf16", "B": B, "K": K, "V": V,
                   "D": D, "temperature": w.T, "positions_per_step": w.positions,
                   "input_sets": 1, "weight_layout": "packed once before timing"},
        "roofline": {"bound": "mfma", "kernel": "lm_head", "achieved": flops / k_us / 1e6,
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": flops / k_us / 1e6 / 2500.0,
                     "traffic": measured_traffic(LM_HEAD_TRAFFIC),
                     "launch_us": k_us, "flops_per_launch": flops,
                     "hbm_gbps": hbm_bytes / k_us / 1e3, "hbm_bytes_per_launch": hbm_bytes},
        "reference_gemm": {"what": "torch.matmul (hipBLASLt) on the same row-major bf16 "
                                   "operands: logits only, no statistics; context",
                           "us_per_launch": blas_us, "tflops": flops / blas_us / 1e6},
    }
    if not args.no_cpu_baseline:
        # the oracle on whole requests: its LM-head rows in float64, then verify
        log(f"timing the oracle for about {args.cpu_seconds:.0f} s")
        t_total, positions, reqs = 0.0, 0, 0
        b = 0
        while t_total < args.cpu_seconds and b < B:
            t1 = time.perf_counter()
            tb = OL.lm_head_target_bits(w.hidden[b:b + 1], w.weight)
            O.verify(tb, w.draft[b:b + 1], w.draft_tokens[b:b + 1], w.draft_len[b:b + 1],
                     w.u[b:b + 1], w.u_final[b:b + 1], w.T, 0, 1.0, w.eos_id, "bf16")
            t_total += time.perf_counter() - t1
            positions += int(w.draft_len[b])
            reqs += 1
            b += 1
        result["cpu_baseline"] = {
            "value": positions / t_total, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"{reqs} requests of the same workload (LM-head rows in float64 numpy, "
                      f"then the verification), {t_total:.1f} s"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=None,
                    help="input sets rotated through (default 4; 1 for workload 4, 2.6 GB each)")
    ap.add_argument("--workload", type=int, choices=[1, 2, 3, 4, 5], default=WORKLOAD,
                    help="synthetic workload of the verify op (3, the default, is the headline)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle timing budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", choices=["verify", "sample", "lm_head", "rates"], default="verify",
                    help="verify: the verification step (default, the headline); sample: the "
                         "draft-side draw of the same workload (256 draft rows); lm_head: the "
                         "verification fused with a D=4096 target LM head; rates: the "
                         "acceptance diagnostics of the same workload; the last three are "
                         "reported for reference")
    ap.add_argument("--top-k", type=int, default=None,
                    help="override the verify workload's top-k (0 = off); reported separately")
    ap.add_argument("--top-p", type=float, default=None,
                    help="override the verify workload's top-p (1.0 = off); reported separately")
    ap.add_argument("--batch", type=int, default=None,
                    help="override the verify workload's batch size; reported separately")
    ap.add_argument("--small-batch-limit", type=int, default=None,
                    help="set the library's small-batch limit (B (K+1) ceil(V/2048) up to which "
                         "unfiltered calls take the one-kernel tail; 0 = never)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "runs on one GPU only; --gpus must be 1"}))
        log("multi-GPU runs are not implemented: the path would shard over requests "
            "with no communication (see the design notes); run with --gpus 1")
        sys.exit(2)

    if args.sets is None:
        args.sets = 1 if args.workload == 4 else 4
    if args.op != "verify" and (args.workload != WORKLOAD or args.top_k is not None
                                or args.top_p is not None or args.batch is not None):
        log("--workload, --top-k, --top-p and --batch apply to the verify op only")
        sys.exit(2)
    if args.op == "sample":
        return bench_sample(args)
    if args.op == "lm_head":
        return bench_lm_head(args)
    if args.op == "rates":
        return bench_rates(args)

    import torch
    from speculative_decoding_sampling_amd import binding
    from speculative_decoding_sampling_amd.build import LIB
    from speculative_decoding_sampling_amd.workloads import (WORKLOADS, make_workload, upload,
                                                             uniforms)

    if not os.path.exists(LIB):
        from speculative_decoding_sampling_amd.build import build
        build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = args.workload
    spec = dict(WORKLOADS[wl])
    if args.small_batch_limit is not None:
        binding.set_small_batch_limit(args.small_batch_limit)
    if args.batch is not None:
        # another batch size of the same workload: a separate line
        spec["B"] = args.batch
        spec["name"] = f"B{args.batch}_" + spec["name"].split("_", 1)[1]
    overridden = args.top_k is not None or args.top_p is not None or args.batch is not None
    if args.top_k is not None or args.top_p is not None:
        # the same logits under other filter settings: a separate line, never
        # the headline
        if args.top_k is not None:
            spec["top_k"] = args.top_k
        if args.top_p is not None:
            spec["top_p"] = args.top_p
        base = spec["name"].split("_topk")[0]
        spec["name"] = base + "".join(
            f"_{n}{v:g}" for n, v, off in (("topk", spec["top_k"], 0), ("topp", spec["top_p"], 1.0))
            if v != off)
    filtered = 0 < spec["top_k"] < spec["V"] or spec["top_p"] < 1.0
    sets, hosts = [], []
    for i in range(args.sets):
        t0 = time.perf_counter()
        seed = 1000 + wl + 100 * i
        if filtered:
            # placeholder drafts, replaced below by draws from the processed
            # draft rows made on the GPU by specv_sample
            w = make_workload(wl, seed=seed, B=spec["B"], draft_sampler=lambda z, T, k, p, x: 0,
                              top_k=spec["top_k"], top_p=spec["top_p"])
        else:
            w = make_workload(wl, seed=seed, B=spec["B"], top_k=spec["top_k"], top_p=spec["top_p"])
        hosts.append(w)
        a = upload(w, dev)
        if filtered:
            R = w.B * w.K
            ud = torch.from_numpy(uniforms(np.random.default_rng(seed + 7), R)).to(dev)
            tok = binding.sample(a["draft_logits"].reshape(R, w.V), ud, w.T, w.top_k, w.top_p)
            a["draft_tokens"] = tok.reshape(w.B, w.K).contiguous()
            w.draft_tokens = a["draft_tokens"].cpu().numpy()
            assert np.all((w.draft_tokens >= 0) & (w.draft_tokens < w.V))
        a["out_tokens"] = torch.empty((w.B, w.K + 1), dtype=torch.int32, device=dev)
        a["n_emitted"] = torch.empty((w.B,), dtype=torch.int32, device=dev)
        sets.append(a)
        log(f"input set {i}: {w.algorithmic_bytes / 1e6:.1f} MB needed rows, "
            f"{w.positions} positions ({time.perf_counter() - t0:.1f} s to generate)")
    w0 = hosts[0]
    # per-step means over the sets the timed steps cycle through (the sets
    # differ only where draft lengths are ragged)
    positions = float(np.mean([hosts[i % len(hosts)].positions for i in range(args.steps)]))
    alg_bytes = float(np.mean([hosts[i % len(hosts)].algorithmic_bytes
                               for i in range(args.steps)]))
    if positions.is_integer() and alg_bytes.is_integer():
        positions, alg_bytes = int(positions), int(alg_bytes)

    stream = torch.cuda.current_stream(dev)
    ldt = sets[0]["target_logits"].dtype
    ws = torch.empty(binding.workspace_bytes(w0.B, w0.K, w0.V, ldt, w0.top_k, w0.top_p),
                     dtype=torch.uint8, device=dev)

    def step(i, events=None):
        binding.verify(**sets[i % len(sets)], workspace=ws, stream=stream, events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # Timed region: K steps bracketed by synchronisation.
    ev = HipEvents(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev.lib.hipEventRecord(ev.arr[0], stream.cuda_stream)
    for i in range(args.steps):
        step(i)
    ev.lib.hipEventRecord(ev.arr[1], stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev.elapsed_ms(0, 1) / args.steps
    ev.close()
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step "
        f"(host wall {wall / args.steps * 1e6:.2f} us/step)")

    # Host enqueue cost alone: a short burst right after a sync, timed on the
    # host before the GPU could back-pressure the launches.
    torch.cuda.synchronize()
    n_burst = 8
    h0 = time.perf_counter()
    for i in range(n_burst):
        step(i)
    host_us = (time.perf_counter() - h0) / n_burst * 1e6
    torch.cuda.synchronize()
    log(f"host enqueue {host_us:.2f} us/call")

    # Single-call durations: one event before each call and one after the last.
    evc = HipEvents(args.steps + 1)
    torch.cuda.synchronize()
    for i in range(args.steps):
        evc.lib.hipEventRecord(evc.arr[i], stream.cuda_stream)
        step(i)
    evc.lib.hipEventRecord(evc.arr[args.steps], stream.cuda_stream)
    torch.cuda.synchronize()
    call_us = np.array([evc.elapsed_ms(i, i + 1) for i in range(args.steps)]) * 1e3
    evc.close()
    p10, med, p90 = (float(x) for x in np.percentile(call_us, [10, 50, 90]))
    log(f"single calls: median {med:.2f} us, p10 {p10:.2f}, p90 {p90:.2f}")

    # Per-kernel durations: the same steps through the timing entry point.
    names = binding.stage_names(binding.path_kind(w0.B, w0.K, w0.V, w0.top_k, w0.top_p))
    nst = len(names)
    evs = [HipEvents(nst + 1) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, events=evs[i].arr)
    torch.cuda.synchronize()
    stage_ms = np.array([[e.elapsed_ms(j, j + 1) for j in range(nst)] for e in evs])
    timed_total = float(np.mean([e.elapsed_ms(0, nst) for e in evs]))
    for e in evs:
        e.close()
    stage_us = {n: float(stage_ms[:, j].mean() * 1e3) for j, n in enumerate(names)}
    log("stage means (us): " + ", ".join(f"{k}={v:.2f}" for k, v in stage_us.items())
        + f"; evented step {timed_total * 1e3:.2f} us")

    # Result sanity: every request emitted a legal count.
    n = sets[0]["n_emitted"].cpu().numpy()
    assert np.all((n >= 1) & (n <= w0.draft_len + 1)), n

    # Context for the roofline: what a plain device copy of 512 MiB reaches on
    # this box (bytes read + written per second), timed like the steps.  Not
    # in counter runs, whose calibration copies are told apart by kernel name.
    copy_gbps = None
    if not args.copy_calibration_mib:
        cal_bytes = 512 << 20
        csrc = torch.empty(cal_bytes // 4, dtype=torch.float32, device=dev).normal_()
        cdst = torch.empty_like(csrc)
        cdst.copy_(csrc)
        evm = HipEvents(2)
        torch.cuda.synchronize()
        evm.lib.hipEventRecord(evm.arr[0], stream.cuda_stream)
        for _ in range(10):
            cdst.copy_(csrc)
        evm.lib.hipEventRecord(evm.arr[1], stream.cuda_stream)
        torch.cuda.synchronize()
        copy_gbps = 2 * cal_bytes * 10 / (evm.elapsed_ms(0, 1) * 1e-3) / 1e9
        evm.close()
        del csrc, cdst
        log(f"plain 512 MiB device copy: {copy_gbps:.0f} GB/s (read + write)")

    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).normal_()
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 copies of {args.copy_calibration_mib} MiB")

    if filtered or len(names) == 1:
        # The dominant kernel is the path's first pass, the top-k candidate
        # pass or the radix select (each reads every needed row), or the
        # small-batch path's one kernel; its duration is the per-call stage
        # mean above.
        dominant = names[0]
        k1_us = stage_us[dominant]
        traffic = measured_traffic(TRAFFIC.get(spec["name"]))
        log(f"{dominant}: {k1_us:.2f} us/launch (stage mean)")
    else:
        # The dominant kernel alone, for the roofline: a burst of row-statistics
        # launches cycling over the input sets between two events on the stream.
        reps = max(40, args.steps)
        evb = HipEvents(2)
        torch.cuda.synchronize()
        binding.bench_row_stats(sets, ws, reps, w0.T, stream, evb.arr[0], evb.arr[1])
        torch.cuda.synchronize()
        dominant = "row_stats"
        k1_us = evb.elapsed_ms(0, 1) / reps * 1e3
        burst_bytes = float(np.mean([hosts[i % len(hosts)].algorithmic_bytes
                                     for i in range(reps)]))
        # the counters were taken on the headline workload's launch
        traffic = measured_traffic(TRAFFIC.get(spec["name"])) if not overridden else None
        evb.close()
        log(f"row_stats alone: {k1_us:.2f} us/launch over {reps} launches")
    if filtered or len(names) == 1:
        burst_bytes = alg_bytes
    achieved = burst_bytes / (k1_us * 1e-6) / 1e9
    step_gbps = alg_bytes / (ms_per_step * 1e-3) / 1e9
    metric = METRIC if wl == WORKLOAD else (
        f"verified draft positions/sec and achieved HBM GB/s (% of peak), {spec['name']}")
    result = {
        "metric": metric,
        "value": positions / (ms_per_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+f64",
        "data": "synthetic",
        "config": {"workload": spec["name"], "B": w0.B, "K": w0.K, "V": w0.V,
                   "logits": w0.dtype, "temperature": float(w0.T), "top_k": int(w0.top_k),
                   "top_p": float(w0.top_p), "input_sets": args.sets,
                   "positions_per_step": positions, "algorithmic_bytes_per_step": alg_bytes},
        "us_per_call": {"median": med, "p10": p10, "p90": p90},
        "host_us_per_call": host_us,
        "hbm_gbps_whole_step": step_gbps,
        "hbm_frac_whole_step": step_gbps / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "launch_us": k1_us,
                     "bytes_per_launch": burst_bytes},
        "stages_us": stage_us,
        "copy_512mib_gbps_read_plus_write": copy_gbps,
    }
    if not args.no_cpu_baseline:
        log(f"timing the oracle for about {args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(w0, args.cpu_seconds,
                                              group=8 if wl == 4 else None,
                                              tokens_from_gpu=filtered)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
