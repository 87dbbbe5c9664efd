"""EFLA fwd+bwd throughput on one MI355X.

One step = efla_fwd (saving chunk factors and states) + efla_bwd (reading them) over
the 1.3B-layer workload: B=4, H=16, T=2048, d_k=d_v=128, bf16 inputs, fp32
accumulation, synthetic seeded inputs already resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
  python bench.py --all-configs [--out FILE]   (per-workload table: GPU times and roofline
                                                 fractions, fp64 oracle time and error)
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


def method_model(dk, dv, e, C=CHUNK):
    """What the method itself must move and compute per token-head: bytes of q, k, v, beta in
    and o out (forward); q, k, v, beta, dO in and dq, dk, dv, dbeta out (backward); flops of
    the chunkwise form's dense tiles (forward: W S, U~, Q S, masked Q K^T and its product, the
    state update, the UT transform; backward about 2.5x that). e = bytes per element.
    Returns dict(fwd_bytes, bwd_bytes, fwd_flops, bwd_flops)."""
    return dict(fwd_bytes=e * (2 * dk + 2 * dv + 1), bwd_bytes=e * (4 * dk + 3 * dv + 2),
                fwd_flops=6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3,
                bwd_flops=14 * dk * dv + 2 * C * (8 * dk + 5 * dv) + 4 * C * C / 3)


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
    (2 per multiply-add). bf16 problems (e = 2) keep X and the column scales alpha~ (fp32, one
    per token) in place of W and U: the scans form U~ = X (diag(alpha~) (V - K S)) and
    W^T dU~ = K^T diag(alpha~) X^T dU~ themselves, and the forward scan forms M = tril(Q K^T)
    from its Q and K tiles (writing it out for the backward); fp32 problems (e = 4) read W and
    U, and M from the UT kernel."""
    xf = e == 2
    if name == "ut_fwd":
        if xf:                # K, beta -> X = (I + A)^-1, alpha~
            b = e * (C * dk + C) + e * C * C + 4 * C
            f = C * C * dk + C ** 3 / 3
        else:                 # Q, K, V, beta -> W, U, M, X
            b = e * (2 * C * dk + C * dv + C) + e * (C * dk + C * dv + 2 * C * C)
            f = 3 * C * C * dk + C * C * dv + C ** 3 / 3
    elif name == "scan_fwd":
        if xf:                # Q, K, X, V, alpha~ -> O, U~, S_c, M = tril(QK^T)
            b = e * (2 * C * dk + C * dv + C * C) + 4 * C + e * (2 * C * dv + dk * dv + C * C)
            f = 6 * C * dk * dv + 2 * C * C * dv + C * C * dk
        else:                 # Q, K, W, U, M -> O, U~, S_c
            b = e * (3 * C * dk + C * dv + C * C) + e * (2 * C * dv + dk * dv)
            f = 6 * C * dk * dv + C * C * dv
    elif name == "scan_bwd":
        if xf:                # Q, K, X, M, dO, alpha~ -> dU~, dS_c
            b = e * (2 * C * dk + 2 * C * C + C * dv) + 4 * C + e * (C * dv + dk * dv)
            f = 6 * C * dk * dv + 2 * C * C * dv
        else:                 # Q, K, W, M, dO -> dU~, dS_c
            b = e * (3 * C * dk + C * C + C * dv) + e * (C * dv + dk * dv)
            f = 6 * C * dk * dv + C * C * dv
    elif name == "chunk_bwd":  # Q, K, V, dO, U~, dU~, beta, S_c, dS_c, X -> dQ, dK, dV, dbeta
        b = e * (2 * C * dk + 4 * C * dv + C + 2 * dk * dv + C * C) + e * (2 * C * dk + C * dv + C)
        f = 6 * C * dk * dv + 7 * C * C * dk + 3 * C * C * dv + 2 * C ** 3 / 3
    else:
        return 0.0, 0.0
    return float(b), float(f)


def _code_only(text):
    """C++ source without its comments and blank lines (string and character literals kept), so
    that edits to comments leave a kernel's hash unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(ch)
            i += 1
    return "\n".join(l.rstrip() for l in "".join(out).splitlines() if l.strip())


def _source_sha(name):
    """Hash of the code (comments excluded) of the sources a kernel is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(name, []):
        with open(os.path.join(ROOT, "delta_rule_sequence_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
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

    import gzip

    def per_kernel(path, counter):  # kernel symbol -> (mean per dispatch, dispatches)
        vals = collections.defaultdict(list)
        opener = gzip.open if path.endswith(".gz") else open
        for r in csv.DictReader(opener(path, "rt")):
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


def _kernel_label(mangled):
    """efla kernel symbol -> 'name<args>' (bf16/f32, integers, T/F); other symbols unchanged."""
    import re
    m = re.match(r"_ZN4efla\d+(\w+?)_kernelI", mangled)
    if not m:
        return mangled[:60]
    rest, args = mangled[m.end():], []
    while rest and rest[0] != "E":
        t = re.match(r"DF16b|f|Li(-?\d+)E|Lb([01])E", rest)
        if not t:
            break
        tok = t.group(0)
        args.append("bf16" if tok == "DF16b" else "f32" if tok == "f" else
                    t.group(1) if t.group(1) is not None else "TF"[1 - int(t.group(2))])
        rest = rest[t.end():]
    return "%s<%s>" % (m.group(1), ",".join(args))


def trace_summary(path):
    """Markdown table of a rocprofv3 kernel trace (kernel_trace.csv, or .csv.gz): dispatches
    grouped by kernel instance and grid size, with count and average / min / max duration."""
    import csv
    import gzip
    import collections
    opener = gzip.open if path.endswith(".gz") else open
    groups = collections.OrderedDict()
    with opener(path, "rt") as f:
        for r in csv.DictReader(f):
            wgs = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            key = (_kernel_label(r["Kernel_Name"]), wgs, int(r["Workgroup_Size_X"]))
            groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | workgroups x threads | calls | avg us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for (name, wgs, wgsz), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        if len(d) < 2 and "efla" not in name and "<" not in name:
            continue
        print("| %s | %d x %d | %d | %.1f | %.1f | %.1f |" % (name, wgs, wgsz, len(d), sum(d) / len(d),
                                                          min(d), max(d)))


def host_info():
    """Host cores available to this process, CPU model and BLAS threads (the oracle's numpy)."""
    import numpy  # noqa: F401  (loads the BLAS library threadpoolctl reports)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import threadpoolctl
        blas = [{"api": d.get("internal_api"), "threads": d.get("num_threads")}
                for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        pass
    return {"host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": model, "blas": blas}


def timed_oracle(fn):
    """Run fn once; returns (result, wall seconds, threads it kept busy = CPU time / wall)."""
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    out = fn()
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    return out, wall, max(1, int(round(cpu / wall)))


def cpu_baseline():
    """The fp64 oracle on one step of the workload itself (all 4 batch rows x 16 heads x 2048
    tokens), forward and backward: about 10 s of host time."""
    from oracle import efla_oracle as O
    from workloads import make_inputs, workload
    w = workload(2)
    inp = make_inputs(w)

    def step():
        O.forward(inp["q"], inp["k"], inp["v"], inp["beta"])
        O.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["do"])
    _, wall, cores = timed_oracle(step)
    out = {"value": w.B * w.T / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": "one full step of the B=4,H=16,T=2048,d=128 workload (16 heads x 8192 "
                     "tokens), fp64 numpy token recurrence fwd+bwd, %.1f s wall; cores = threads "
                     "it kept busy (CPU time / wall)" % wall}
    out.update(host_info())
    return out


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

    run = event_timer(torch, torch.cuda.current_stream())

    def timed(f):
        prewarm(torch, f, 0.3)
        return run(f, iters)

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
                    "fwd_bwd_tokens_per_s": round(w.B * w.T / (ms_step * 1e-3), 1),
                    "fwd_kernels_avg_ms": kernel_avgs(
                        E, lambda: E.efla_fwd(q, k, v, beta, 1.0, None, False, ws, o=o, segments=segs), iters)[0],
                    "fwd_bwd_kernels_avg_ms": kernel_avgs(E, step, iters)[0]}
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


def prewarm(torch, f, seconds=0.5):
    """Runs f repeatedly for about `seconds` (untimed): after idle time the GPU needs some tens
    of milliseconds of work before its step time settles (clock and power ramp)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            f()
        torch.cuda.synchronize()


def event_timer(torch, stream):
    """Times a callable over n calls with two HIP events on `stream`; returns ms per call."""
    def run(f, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            f()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / n
    return run


def kernel_avgs(E, f, n):
    """Per-kernel average ms of n calls of f, from the library's launch events."""
    import torch
    E.profile_reset()
    E.profile_enable(True)
    for _ in range(n):
        f()
    torch.cuda.synchronize()
    prof = E.profile_read()
    E.profile_enable(False)
    return {k: round(t / max(c, 1), 5) for k, (c, t) in prof.items()}, prof


def euler_ab(torch, step_exact, step_euler, stream, blocks=20, per_block=10):
    """The exact flow against the delta rule on the same tensors and kernels (alpha = beta),
    interleaved: blocks of per_block steps alternate between the two modes (the order flips
    every block), each block timed with events, so both see the same clocks and cache state."""
    run = event_timer(torch, stream)
    for _ in range(3):
        step_exact()
        step_euler()
    ex, eu = [], []
    for i in range(blocks):
        pair = ((step_exact, ex), (step_euler, eu))
        for f, acc in (pair if i % 2 == 0 else pair[::-1]):
            acc.append(run(f, per_block))
    ms_ex, ms_eu = sum(ex) / len(ex), sum(eu) / len(eu)
    return {"steps_each": blocks * per_block, "exact_ms_per_step": round(ms_ex, 4),
            "euler_ms_per_step": round(ms_eu, 4), "exact_over_euler_time": round(ms_ex / ms_eu, 4),
            "block_ratio_min_max": [round(min(a / b for a, b in zip(ex, eu)), 4),
                                    round(max(a / b for a, b in zip(ex, eu)), 4)]}


def all_configs(E, args):
    """Every workload: GPU forward (inference, nothing saved) and forward + backward (the
    training step) times from events, tokens/s, the method-bytes HBM fraction and the
    dense-tile MFMA fraction (peak of the workload's dtype), then the fp64 oracle on the whole
    workload (timed, single process) and the GPU's normwise error against it, per tensor
    (largest over the whole tensor and over the (sequence, head) streams)."""
    import numpy as np
    import torch
    from oracle import efla_oracle as O
    from workloads import make_inputs, workload

    rows = []
    host = host_info()
    for idx in (1, 2, 3, 4, 5):
        w = workload(idx)
        inp = make_inputs(w, with_grad=True)
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        e = 4 if w.dtype == "f32" else 2
        dev = torch.device("cuda:0")
        q, k, v, beta, do = (torch.from_numpy(inp[n]).to(dev, dt) for n in ("q", "k", "v", "beta", "do"))
        cu_np = inp["cu_seqlens"]
        cu = None if cu_np is None else torch.from_numpy(cu_np).to(dev)
        B, H, T, dk = inp["k"].shape
        dv = inp["v"].shape[-1]
        p = E.make_problem(q, k, v, beta, 1.0, cu)
        o = torch.empty_like(v)
        saved = torch.empty(E.efla_saved_bytes(p), dtype=torch.uint8, device=dev)
        ws = torch.empty(max(E.efla_workspace_bytes(p, False), E.efla_workspace_bytes(p, True)),
                         dtype=torch.uint8, device=dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(beta))

        def fwd():
            E.efla_fwd(q, k, v, beta, 1.0, cu, False, ws, o=o)

        def step():
            E.efla_fwd(q, k, v, beta, 1.0, cu, True, ws, o=o, saved=saved)
            E.efla_bwd(q, k, v, beta, do, saved, 1.0, cu, ws, grads=grads)
        run = event_timer(torch, torch.cuda.current_stream())
        n = 20 if B * H * T <= 2 ** 21 else 8
        prewarm(torch, fwd)
        ms_f = run(fwd, n)
        prewarm(torch, step)
        ms_s = run(step, n)
        gpu = {"o": o.float().cpu().numpy()}
        if w.backward:
            gpu.update(zip(("dq", "dk", "dv", "dbeta"), (t.float().cpu().numpy() for t in grads)))
        mm = method_model(dk, dv, e)
        th = B * H * T
        peak_mfma = MFMA_F32_PEAK_TFLOPS if w.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
        row = {"workload": idx, "name": w.name, "B": B, "H": H, "T": T, "d_k": dk, "d_v": dv,
               "dtype": w.dtype, "packed_sequences": None if cu_np is None else len(cu_np) - 1,
               "gpu_fwd_us": round(ms_f * 1e3, 1), "gpu_fwd_bwd_us": round(ms_s * 1e3, 1),
               "fwd_tokens_per_s": round(B * T / (ms_f * 1e-3), 1),
               "fwd_bwd_tokens_per_s": round(B * T / (ms_s * 1e-3), 1),
               "fwd_hbm_frac": round(mm["fwd_bytes"] * th / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "fwd_bwd_hbm_frac": round((mm["fwd_bytes"] + mm["bwd_bytes"]) * th / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "fwd_mfma_frac": round(mm["fwd_flops"] * th / (ms_f * 1e-3) / 1e12 / peak_mfma, 4),
               "fwd_bwd_mfma_frac": round((mm["fwd_flops"] + mm["bwd_flops"]) * th / (ms_s * 1e-3) / 1e12 / peak_mfma, 4),
               "mfma_peak_TFLOPs": peak_mfma}
        del q, k, v, beta, do, o, saved, ws, grads
        torch.cuda.empty_cache()
        print("workload %d: GPU fwd %.1f us, fwd+bwd %.1f us; running the oracle" %
              (idx, row["gpu_fwd_us"], row["gpu_fwd_bwd_us"]), flush=True)
        # the oracle, whole workload, one sequence after the other (what its own loop does)
        spans = [(b, 0, T) for b in range(B)] if cu_np is None else \
            [(0, int(cu_np[i]), int(cu_np[i + 1])) for i in range(len(cu_np) - 1)]
        if cu_np is None:
            spans = [(None, 0, T)]
        ref = {nm: np.zeros(gpu[nm].shape) for nm in gpu}
        t_fwd = t_bwd = 0.0
        cores = 1
        last = time.time()
        for (b, s0, s1) in spans:
            bs = slice(None) if b is None else slice(b, b + 1)
            sl = lambda x: x[bs, :, s0:s1]
            r, wall, c = timed_oracle(lambda: O.forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"])))
            t_fwd += wall
            cores = max(cores, c)
            ref["o"][bs, :, s0:s1] = r[0]
            if w.backward:
                g, wall, c = timed_oracle(lambda: O.backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]),
                                                             sl(inp["beta"]), sl(inp["do"])))
                t_bwd += wall
                cores = max(cores, c)
                for nm in ("dq", "dk", "dv", "dbeta"):
                    ref[nm][bs, :, s0:s1] = g[nm]
            if time.time() - last > 20:
                last = time.time()
                print("  oracle: sequence [%d, %d) done, %.0f s so far" % (s0, s1, t_fwd + t_bwd), flush=True)
        errs = {}
        for nm in gpu:
            per = [O.rel_err(gpu[nm][bs_, h, s0:s1], ref[nm][bs_, h, s0:s1])
                   for (b, s0, s1) in ([(b_, 0, T) for b_ in range(B)] if cu_np is None else spans)
                   for bs_ in [b] for h in range(H)]
            errs[nm] = {"tensor": float("%.3e" % O.rel_err(gpu[nm], ref[nm])),
                        "worst_stream": float("%.3e" % max(per)), "streams": len(per)}
        row.update({"oracle_fwd_s": round(t_fwd, 2), "oracle_fwd_bwd_s": round(t_fwd + t_bwd, 2) if w.backward else None,
                    "oracle_fwd_tokens_per_s": round(B * T / t_fwd, 1),
                    "oracle_fwd_bwd_tokens_per_s": round(B * T / (t_fwd + t_bwd), 1) if w.backward else None,
                    "oracle_threads": cores, "errors_vs_oracle": errs,
                    "tolerance": 1e-4 if w.dtype == "f32" else 2e-2})
        rows.append(row)
        print(json.dumps(row), flush=True)
        del inp, gpu, ref
    out = {"host": host, "workloads": rows}
    print(json.dumps(out), flush=True)
    if args.out:
        with open(args.out, "w") as f:
            json.dump(out, f, indent=1)


def aux_measurements(E, args, torch, np, make_inputs, workload, step, q, k, v, beta, do, o, saved,
                     ws, grads):
    """Everything in the bench line beside the headline: the step as a HIP graph, a cold-cache
    step, the delta-rule A/B, gated EFLA, decode and the long-context workload."""
    B, H, T = q.shape[0], q.shape[1], q.shape[2]
    dk, dv = k.shape[-1], v.shape[-1]
    dev = q.device
    stream = torch.cuda.current_stream()
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
    # replays and eager steps alternate in blocks after a pre-warm, both timed on the host clock
    # around a synchronize, so neither sees the clock ramp that follows the capture
    prewarm(torch, graph.replay)
    graph_t = eager_t = 0.0
    n_blk = max(1, args.steps // 10)
    for blk in range(2 * n_blk):
        f = graph.replay if blk % 2 == 0 else step
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            f()
        torch.cuda.synchronize()
        if blk % 2 == 0:
            graph_t += time.perf_counter() - t0
        else:
            eager_t += time.perf_counter() - t0
    graph_ms = graph_t * 1e3 / (10 * n_blk)
    graph_eager_ms = eager_t * 1e3 / (10 * n_blk)
    del graph

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
    # tensors and kernels with alpha = beta (Euler mode), interleaved with the exact flow, 200
    # steps each whatever --steps is, plus each mode's per-kernel times.
    def step_euler():
        E.efla_fwd(q, k, v, beta, 1.0, None, True, ws, o=o, saved=saved, mode="euler")
        E.efla_bwd(q, k, v, beta, do, saved, 1.0, None, ws, grads=grads, mode="euler")

    euler = euler_ab(torch, step, step_euler, stream)
    euler["exact_kernels_avg_ms"] = kernel_avgs(E, step, 100)[0]
    euler["euler_kernels_avg_ms"] = kernel_avgs(E, step_euler, 100)[0]

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
    gated["kernels_avg_ms"] = kernel_avgs(E, step_gated, args.steps)[0]

    def fwd_pair():
        E.efla_fwd_gated(q, k, v, beta, gate, 1.0, None, False, ws, o=o)
        E.efla_fwd(q, k, v, beta, 1.0, None, False, ws, o=o)
    gated["inference_fwd_kernels_avg_ms"] = kernel_avgs(E, fwd_pair, args.steps)[0]
    gated["gated_fwd_bwd_tokens_per_s"] = round(B * T / (gated["gated_fwd_bwd_ms"] * 1e-3), 1)

    # Recurrent decoding: one token for every (batch row, head), state in fp32.
    state = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=dev)
    q1, k1, v1, b1 = (t[:, :, :1].contiguous() for t in (q, k, v, beta))
    o1 = torch.empty_like(v1)

    def dec():
        E.efla_decode(q1, k1, v1, b1, state, 1.0, o=o1)
    for _ in range(args.warmup):
        dec()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec()
    torch.cuda.synchronize()
    decode_us = (time.perf_counter() - t0) * 1e6 / args.steps
    dec_k = kernel_avgs(E, dec, args.steps)[0]
    dec_kernel_us = 1e3 * sum(dec_k.values())
    # A serving loop without host launch cost: 16 decode calls (one token each) captured into one
    # HIP graph and replayed; time per call.
    decode_graph_us = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            dec()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        dg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dg):
            for _ in range(16):
                dec()
        prewarm(torch, dg.replay, 0.2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dg.replay()
        torch.cuda.synchronize()
        decode_graph_us = (time.perf_counter() - t0) * 1e6 / (16 * args.steps)
        del dg
    except RuntimeError as e:  # reported as null; the rest of the line stands
        print("decode graph not measured: %s" % e, file=sys.stderr)
    state_bytes = 2 * B * H * dk * dv * 4 + B * H * (2 * dk + 2 * dv + 1) * 2  # state in + out, tokens

    # Long context (the pages' long-sequence setting, forward only): B=1, H=16, T=32768. The
    # segment-parallel scan (library's choice of segments) against one sequential chain.
    long_ctx = None if args.no_long_context else long_context(E, make_inputs, workload, args.warmup,
                                                                max(5, args.steps // 5))

    return {"graph_ms": graph_ms, "graph_eager_ms": graph_eager_ms, "cold_ms": cold_ms, "euler": euler, "gated": gated,
            "decode_us": decode_us, "dec_k": dec_k, "dec_kernel_us": dec_kernel_us,
            "decode_graph_us": decode_graph_us,
            "state_bytes": state_bytes, "long_ctx": long_ctx}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the B=1, T=32768 forward (e.g. for per-kernel counter runs)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the benchmark step (no graph, cold-cache, delta-rule, gated, "
                         "decode or long-context parts; for kernel traces and counter runs)")
    ap.add_argument("--long-context-only", action="store_true",
                    help="run only the B=1, T=32768 part and print its JSON (for its kernel trace)")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the benchmark line: every workload's GPU times, roofline "
                         "fractions, fp64 oracle time and error vs the oracle (several minutes)")
    ap.add_argument("--out", default=None, help="--all-configs: also write the table here")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print a rocprofv3 kernel trace grouped by kernel instance and grid, then exit")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store per-kernel HBM traffic from two rocprofv3 --pmc csv files and exit")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
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
    if args.all_configs:
        all_configs(E, args)
        return
    if args.long_context_only:
        print(json.dumps(long_context(E, make_inputs, workload, args.warmup, max(5, args.steps // 5))),
              flush=True)
        return
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

    stream = torch.cuda.current_stream()
    prewarm(torch, step)  # untimed; the measurements below then see the GPU at its steady clocks
    aux = aux_measurements(E, args, torch, np, make_inputs, workload, step, q, k, v, beta, do, o,
                           saved, ws, grads) if not args.headline_only else {}
    # The headline: W untimed warmup steps, then exactly K steps between two synchronizations,
    # after half a second of untimed steps: after idle time (input generation, allocations) or
    # other work (the measurements above) a step needs some 60-80 repetitions to settle at its
    # steady-state time (clock and power ramp, caches), so the timed steps see the GPU as a
    # training loop keeps it.
    prewarm(torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
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
    if aux:
        aux["gated"]["gated_over_ungated_fwd_bwd_time"] = round(aux["gated"]["gated_fwd_bwd_ms"] / ms_per_step, 4)

    # Per-kernel durations: HIP events recorded by the library around each launch, on the
    # stream the kernel runs on, over a second timed region of the same length.
    _, prof = kernel_avgs(E, step, args.steps)

    units = B * H * (T // CHUNK)
    mm = method_model(dk, dv, 2)
    tok_heads = B * H * T
    kernels = {}
    for name, (count, total_ms) in prof.items():
        b, f = kernel_model(name, dk, dv, 2)
        avg = total_ms / max(count, 1)
        kernels[name] = {"avg_ms": round(avg, 5), "launches": count,
                         "interface_GBps": round(b * units / (avg * 1e-3) / 1e9, 1) if b else None,
                         "kernel_model_TFLOPs": round(f * units / (avg * 1e-3) / 1e12, 2) if f else None}
    dom = max((n for n in prof if n in KERNEL_SOURCES), key=lambda n: prof[n][1])
    avg_s = prof[dom][1] / prof[dom][0] * 1e-3
    b_if, f_km = kernel_model(dom, dk, dv, 2)
    # chunk_bwd reads the backward's method inputs and writes its method outputs; a forward
    # kernel would be charged the forward's
    b_meth = (mm["bwd_bytes"] if dom in ("chunk_bwd", "scan_bwd") else mm["fwd_bytes"]) * tok_heads
    ach = b_meth / avg_s / 1e9
    traffic = _stored_traffic(dom, units)
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom, "avg_ms": round(avg_s * 1e3, 5),
                "method_bytes_per_launch": b_meth,
                "method_bytes_per_token_head": mm["bwd_bytes"] if dom in ("chunk_bwd", "scan_bwd") else mm["fwd_bytes"],
                "interface_bytes_per_launch": b_if * units,
                "achieved_interface": round(b_if * units / avg_s / 1e9, 1),
                "frac_interface": round(b_if * units / avg_s / 1e9 / HBM_PEAK_GBS, 4),
                "traffic_over_method": round(traffic / b_meth, 3) if traffic else None,
                "kernel_model_mfma_frac": round(f_km * units / avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    step_bytes = (mm["fwd_bytes"] + mm["bwd_bytes"]) * tok_heads
    step_flops = (mm["fwd_flops"] + mm["bwd_flops"]) * tok_heads
    step_s = ms_per_step * 1e-3
    out = {
        "metric": "EFLA fwd+bwd tokens/s at B=4,H=16,T=2048,d=128 bf16; % of MFMA peak",
        "value": round(B * T / step_s, 1),
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
        # the whole step against the method's own bytes and dense-tile flops (q, k, v, beta, o,
        # dO and the gradients; 6 d_k d_v + ... per token-head, forward and backward)
        "step_method_bytes": step_bytes,
        "step_hbm_frac": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_method_flops": step_flops,
        "step_mfma_TFLOPs": round(step_flops / step_s / 1e12, 2),
        "step_mfma_frac": round(step_flops / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernels": kernels,
        "roofline": roofline,
    }
    if aux:
        graph_ms, cold_ms = aux["graph_ms"], aux["cold_ms"]
        out.update({
            "hip_graph": {"ms_per_step": round(graph_ms, 4),
                          "tokens_per_s": round(B * T / (graph_ms * 1e-3), 1),
                          "eager_ms_per_step_interleaved": round(aux["graph_eager_ms"], 4)},
            "cold_cache": {"median_ms_per_step": round(cold_ms[len(cold_ms) // 2], 4),
                           "tokens_per_s": round(B * T / (cold_ms[len(cold_ms) // 2] * 1e-3), 1),
                           "steps": len(cold_ms)},
            "euler_mode": aux["euler"],
            "decode": {"us_per_call": round(aux["decode_us"], 2),
                       "graph_us_per_call": None if aux["decode_graph_us"] is None else round(aux["decode_graph_us"], 2),
                       "kernel_us": round(aux["dec_kernel_us"], 2),
                       "kernels_avg_ms": aux["dec_k"], "tokens_per_call": B, "token_heads_per_call": B * H,
                       "hbm_bytes_per_call": aux["state_bytes"],
                       "kernel_hbm_frac": round(aux["state_bytes"] / (aux["dec_kernel_us"] * 1e-6) / 1e9
                                                / HBM_PEAK_GBS, 4)},
            "gated": aux["gated"],
            "long_context": aux["long_ctx"],
        })
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
