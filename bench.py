"""EFLA fwd+bwd throughput on one MI355X.

One step = efla_fwd (saving chunk factors and states) + efla_bwd (reading them) over
the 1.3B-layer workload: B=4, H=16, T=2048, d_k=d_v=128, bf16 inputs, fp32
accumulation, synthetic seeded inputs already resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3
CHUNK = 64

# Kernel source files, for matching stored counter readings to the current code.
KERNEL_SOURCES = {
    "ut_fwd": ["efla_ut.hip", "efla_device.hpp"],
    "scan_fwd": ["efla_scan_fwd.hip", "efla_device.hpp"],
    "scan_bwd": ["efla_scan_bwd.hip", "efla_device.hpp"],
    "chunk_bwd": ["efla_chunk_bwd.hip", "efla_device.hpp"],
}


def kernel_model(name, dk, dv, e, C=CHUNK):
    """Algorithmic HBM bytes and flops of one kernel per (chunk, head) unit.

    Bytes are the tensors the kernel must read and write at its interface (each once);
    flops count the tile contractions the method needs, triangular factors at half size
    (2 per multiply-add)."""
    if name == "ut_fwd":      # Q, K, V, beta -> W, U, M = tril(QK^T), X = (I + A)^-1
        b = e * (2 * C * dk + C * dv + C) + e * (C * dk + C * dv + 2 * C * C)
        f = 3 * C * C * dk + C * C * dv + C ** 3 / 3
    elif name == "scan_fwd":  # Q, K, W, U, M -> O, U~, S_c
        b = e * (3 * C * dk + C * dv + C * C) + e * (2 * C * dv + dk * dv)
        f = 6 * C * dk * dv + C * C * dv
    elif name == "scan_bwd":  # Q, K, W, M, dO -> dU~, dS_c
        b = e * (3 * C * dk + C * C + C * dv) + e * (C * dv + dk * dv)
        f = 6 * C * dk * dv + C * C * dv
    elif name == "chunk_bwd":  # Q, K, V, dO, U~, dU~, beta, S_c, dS_c, X -> dQ, dK, dV, dbeta
        b = e * (2 * C * dk + 4 * C * dv + C + 2 * dk * dv + C * C) + e * (2 * C * dk + C * dv + C)
        f = 6 * C * dk * dv + 7 * C * C * dk + 3 * C * C * dv + 2 * C ** 3 / 3
    else:
        return 0.0, 0.0
    return float(b), float(f)


def _source_sha(name):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(name, []):
        with open(os.path.join(ROOT, "delta_rule_sequence_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _stored_traffic(name, units):
    """HBM bytes per launch from profiles/counters_<kernel>.json when it matches this code."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_sha") != _source_sha(name):
        return None
    return float(c["hbm_bytes_per_launch"])


def ingest_counters(fetch_csv, write_csv, probe_mib):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) into
    HBM bytes per launch for each EFLA kernel, scaled by what the same counters read for
    the plain copy of probe_mib MiB, and store them as profiles/counters_<kernel>.json."""
    import csv
    import collections

    def per_kernel(path, counter):  # kernel symbol -> (mean per dispatch, dispatches)
        vals = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = probe_mib * 1024.0
    cf = [v[0] for k, v in fetch.items() if "copyBuffer" in k]
    cw = [v[0] for k, v in write.items() if "copyBuffer" in k]
    fetch_scale, write_scale = copy_kib / cf[0], copy_kib / cw[0]

    def step_instance(d, name):  # the template instance the timed step launches most often
        cand = [(v[1], v[0]) for k, v in d.items()
                if "efla" in k and (name + "_kernel" in k or name + "_dma_kernel" in k)]
        return [max(cand)[1]] if cand else []

    out = {}
    for name in KERNEL_SOURCES:
        fk = step_instance(fetch, name)
        wk = step_instance(write, name)
        if not fk or not wk:
            continue
        rec = {"kernel": name, "source_sha": _source_sha(name),
               "fetch_kib_per_dispatch": round(fk[0], 2), "write_kib_per_dispatch": round(wk[0], 2),
               "fetch_scale": round(fetch_scale, 5), "write_scale": round(write_scale, 5),
               "copy_probe_mib": probe_mib,
               "hbm_bytes_per_launch": round((fk[0] * fetch_scale + wk[0] * write_scale) * 1024.0)}
        with open(os.path.join(ROOT, "profiles", "counters_%s.json" % name), "w") as f:
            json.dump(rec, f, indent=1)
        out[name] = rec
    print(json.dumps(out, indent=1))


def cpu_baseline():
    """The fp64 oracle on one step of the workload itself (all 4 batch rows x 16 heads x 2048
    tokens), forward and backward: about 10 s of host time."""
    from oracle import efla_oracle as O
    from workloads import make_inputs, workload
    w = workload(2)
    inp = make_inputs(w)
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    O.forward(inp["q"], inp["k"], inp["v"], inp["beta"])
    O.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["do"])
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    cores = max(1, int(round(cpu / wall)))
    return {"value": w.B * w.T / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "one full step of the B=4,H=16,T=2048,d=128 workload (16 heads x 8192 "
                      "tokens), fp64 numpy token recurrence fwd+bwd, %.1f s wall" % wall}


def long_context(E, make_inputs, workload, warmup, iters):
    """B=1, H=16, T=32768, d=128 bf16 (few sequence-head pairs, long sequences): the forward
    alone (inference), and forward + backward (training step), each with the segment-parallel
    scans (segments chosen by the library) and with a single sequential chain per sequence."""
    import torch
    w = workload(3)
    inp = make_inputs(w, with_grad=True)
    q, k, v, beta, do = (torch.from_numpy(inp[n]).to("cuda", torch.bfloat16)
                         for n in ("q", "k", "v", "beta", "do"))
    o = torch.empty_like(v)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(beta))
    res = {"workload": "efla_fwd_B1_H16_T32768_d128_bf16"}
    lay = None

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(iters):
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / iters

    for segs, key in ((0, "segmented"), (1, "sequential")):
        p = E.make_problem(q, k, v, beta, segments=segs)
        ws = torch.empty(max(E.efla_workspace_bytes(p, False), E.efla_workspace_bytes(p, True)),
                         dtype=torch.uint8, device="cuda")
        saved = torch.empty(E.efla_saved_bytes(p), dtype=torch.uint8, device="cuda")
        ms = timed(lambda: E.efla_fwd(q, k, v, beta, 1.0, None, False, ws, o=o, segments=segs))

        def step():
            E.efla_fwd(q, k, v, beta, 1.0, None, True, ws, o=o, saved=saved, segments=segs)
            E.efla_bwd(q, k, v, beta, do, saved, 1.0, None, ws, grads=grads, segments=segs)

        ms_step = timed(step)
        res[key] = {"ms_fwd": round(ms, 4), "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
                    "ms_fwd_bwd": round(ms_step, 4),
                    "fwd_bwd_tokens_per_s": round(w.B * w.T / (ms_step * 1e-3), 1)}
        if segs == 0:
            lay = E.efla_workspace_bytes(p, False) - E.efla_workspace_bytes(
                E.make_problem(q, k, v, beta, segments=1), False)
        del ws, saved
    # segments the library chose: extra workspace / (4 H dk (2 dv + dk)) bytes per segment
    res["segments"] = int(lay // (4 * w.H * w.dk * (2 * w.dv + w.dk)))
    res["speedup"] = round(res["sequential"]["ms_fwd"] / res["segmented"]["ms_fwd"], 3)
    res["fwd_bwd_speedup"] = round(res["sequential"]["ms_fwd_bwd"] / res["segmented"]["ms_fwd_bwd"], 3)
    del q, k, v, beta, o, do, grads
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the B=1, T=32768 forward (e.g. for per-kernel counter runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store per-kernel HBM traffic from two rocprofv3 --pmc csv files and exit")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters[0], args.ingest_counters[1], args.copy_probe_mib or 1024)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (got --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import delta_rule_sequence_amd as E
    from workloads import make_inputs, workload

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    E._lib.lib()
    if args.copy_probe_mib > 0:
        # A plain copy of known size: reads and writes copy_probe_mib MiB once each.
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = workload(2)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, beta, do = (torch.from_numpy(inp[n]).to(dev, torch.bfloat16)
                         for n in ("q", "k", "v", "beta", "do"))
    p = E.make_problem(q, k, v, beta)
    o = torch.empty_like(v)
    saved = torch.empty(E.efla_saved_bytes(p), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(E.efla_workspace_bytes(p, False), E.efla_workspace_bytes(p, True)),
                     dtype=torch.uint8, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(beta))

    def step():
        E.efla_fwd(q, k, v, beta, 1.0, None, True, ws, o=o, saved=saved)
        E.efla_bwd(q, k, v, beta, do, saved, 1.0, None, ws, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps

    # The same step captured once into a HIP graph and replayed (every kernel still runs; only
    # the host launches are gone), timed the same way.
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    del graph

    # Per-kernel durations: HIP events recorded by the library around each launch, on the
    # stream the kernel runs on, over a second timed region of the same length.
    E.profile_reset()
    E.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = E.profile_read()
    E.profile_enable(False)

    # Cold last-level cache: before each step a 512 MiB buffer is overwritten (evicting the
    # 256 MB Infinity Cache), and only the step is timed, with events on the same stream.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(max(5, args.steps // 2)):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        cold.append((e0, e1))
    torch.cuda.synchronize()
    cold_ms = sorted(a.elapsed_time(b) for a, b in cold)
    del flush

    # The pages' only efficiency claim: training throughput on par with the delta rule. Same
    # tensors and kernels with alpha = beta (Euler mode), timed the same way.
    def step_euler():
        E.efla_fwd(q, k, v, beta, 1.0, None, True, ws, o=o, saved=saved, mode="euler")
        E.efla_bwd(q, k, v, beta, do, saved, 1.0, None, ws, grads=grads, mode="euler")

    for _ in range(args.warmup):
        step_euler()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_euler()
    torch.cuda.synchronize()
    euler_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # Gated EFLA forward on the same tensors (log-decays log sigmoid(N(3, 1)), bf16) against the
    # ungated forward without a saved buffer (the gated forward is an inference forward).
    gate = torch.from_numpy(-np.logaddexp(0.0, -(np.random.default_rng(5).standard_normal((B, H, T)) + 3.0))
                            .astype(np.float32)).to(dev, torch.bfloat16)
    gated = {}
    for key, f in (("gated", lambda: E.efla_fwd_gated(q, k, v, beta, gate, 1.0, None, False, ws, o=o)),
                   ("ungated", lambda: E.efla_fwd(q, k, v, beta, 1.0, None, False, ws, o=o))):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            f()
        torch.cuda.synchronize()
        gated[key + "_fwd_ms"] = round((time.perf_counter() - t0) * 1e3 / args.steps, 4)
    gated["gated_over_ungated_time"] = round(gated["gated_fwd_ms"] / gated["ungated_fwd_ms"], 4)
    gated["gated_fwd_tokens_per_s"] = round(B * T / (gated["gated_fwd_ms"] * 1e-3), 1)
    # Gated training step: forward saving the backward buffer, then the gated backward.
    ggrads = grads + (torch.empty_like(gate),)

    def step_gated():
        E.efla_fwd_gated(q, k, v, beta, gate, 1.0, None, True, ws, o=o, saved=saved)
        E.efla_bwd_gated(q, k, v, beta, gate, do, saved, 1.0, None, ws, grads=ggrads)

    for _ in range(args.warmup):
        step_gated()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_gated()
    torch.cuda.synchronize()
    gated["gated_fwd_bwd_ms"] = round((time.perf_counter() - t0) * 1e3 / args.steps, 4)
    E.profile_reset()
    E.profile_enable(True)
    for _ in range(args.steps):
        step_gated()
    torch.cuda.synchronize()
    gated["kernels_avg_ms"] = {n: round(t / max(c, 1), 5) for n, (c, t) in E.profile_read().items()}
    E.profile_reset()
    E.profile_enable(True)
    for _ in range(args.steps):
        E.efla_fwd_gated(q, k, v, beta, gate, 1.0, None, False, ws, o=o)
        E.efla_fwd(q, k, v, beta, 1.0, None, False, ws, o=o)
    torch.cuda.synchronize()
    gated["inference_fwd_kernels_avg_ms"] = {n: round(t / max(c, 1), 5) for n, (c, t) in E.profile_read().items()}
    E.profile_enable(False)
    gated["gated_fwd_bwd_tokens_per_s"] = round(B * T / (gated["gated_fwd_bwd_ms"] * 1e-3), 1)
    gated["gated_over_ungated_fwd_bwd_time"] = round(gated["gated_fwd_bwd_ms"] / ms_per_step, 4)

    # Recurrent decoding: one token for every (batch row, head), state in fp32.
    state = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=dev)
    q1, k1, v1, b1 = (t[:, :, :1].contiguous() for t in (q, k, v, beta))
    o1 = torch.empty_like(v1)
    for _ in range(args.warmup):
        E.efla_decode(q1, k1, v1, b1, state, 1.0, o=o1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        E.efla_decode(q1, k1, v1, b1, state, 1.0, o=o1)
    torch.cuda.synchronize()
    decode_us = (time.perf_counter() - t0) * 1e6 / args.steps

    # Long context (the pages' long-sequence setting, forward only): B=1, H=16, T=32768. The
    # segment-parallel scan (library's choice of segments) against one sequential chain.
    long_ctx = None if args.no_long_context else long_context(E, make_inputs, workload, args.warmup,
                                                                max(5, args.steps // 5))

    units = B * H * (T // CHUNK)
    kernels = {}
    for name, (count, total_ms) in prof.items():
        b, f = kernel_model(name, dk, dv, 2)
        avg = total_ms / max(count, 1)
        kernels[name] = {"avg_ms": round(avg, 5), "launches": count,
                         "alg_GBps": round(b * units / (avg * 1e-3) / 1e9, 1) if b else None,
                         "alg_TFLOPs": round(f * units / (avg * 1e-3) / 1e12, 2) if f else None}
    dom = max((n for n in prof if n in KERNEL_SOURCES), key=lambda n: prof[n][1])
    b, f = kernel_model(dom, dk, dv, 2)
    avg_s = prof[dom][1] / prof[dom][0] * 1e-3
    ach = b * units / avg_s / 1e9
    traffic = _stored_traffic(dom, units)
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom, "avg_ms": round(avg_s * 1e3, 5),
                "mfma_TFLOPs": round(f * units / avg_s / 1e12, 2),
                "mfma_frac": round(f * units / avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}

    step_flops = sum(kernel_model(n, dk, dv, 2)[1] for n in KERNEL_SOURCES) * units
    out = {
        "metric": "EFLA fwd+bwd tokens/s at B=4,H=16,T=2048,d=128 bf16; % of MFMA peak",
        "value": round(B * T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "efla_fwd_bwd_B4_H16_T2048_d128_bf16", "B": B, "H": H, "T": T,
                   "d_k": dk, "d_v": dv, "chunk": CHUNK, "tokens_per_step": B * T},
        "event_ms_per_step": round(ev_ms, 4),
        "step_mfma_frac": round(step_flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernels": kernels,
        "roofline": roofline,
        "hip_graph": {"ms_per_step": round(graph_ms, 4),
                      "tokens_per_s": round(B * T / (graph_ms * 1e-3), 1)},
        "cold_cache": {"median_ms_per_step": round(cold_ms[len(cold_ms) // 2], 4),
                       "tokens_per_s": round(B * T / (cold_ms[len(cold_ms) // 2] * 1e-3), 1),
                       "steps": len(cold_ms)},
        "euler_mode": {"ms_per_step": round(euler_ms, 4),
                       "exact_over_euler_time": round(ms_per_step / euler_ms, 4)},
        "decode": {"us_per_call": round(decode_us, 2), "tokens_per_call": B,
                   "state_MB": round(B * H * dk * dv * 4 / 1e6, 2)},
        "gated": gated,
        "long_context": long_ctx,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
