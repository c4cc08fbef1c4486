"""Benchmark of carve_chunk_fwd on one MI355X.

One step = one forward pass of the CARVE layer over the batch (every stage of
the path: gate prep, gated Grams and triangular inverse, W/U, the serial state
pass, output and chunk mean), writing o, the final state and the final mean.
Default workload: B=4, H=12, T=2048, d_k=d_v=64, L=64, bf16 inputs with fp32
accumulation, no content projection (seeded synthetic data); --workload picks
another of the named shapes.

Prints one JSON line. The timed steps run back to back and rotate through
several copies of the inputs, so that no step finds its inputs in the 256 MB
Infinity Cache. `roofline` covers one call of the layer (its kernels run back
to back on one stream): algorithmic bytes per call over the GPU time per call,
taken from one pair of HIP events recorded on that stream around the timed
steps; the same call timed on one input copy, and single calls after a 512 MB
cache flush, are reported beside it. `mfma` is the matrix-core roofline of the
same call (algorithmic FLOPs over the same time, against the dense peak of the
input type), with the committed rocprofv3 matrix-core counters when they match
the kernel sources. `cpu_baseline` is the float64 oracle timed on this host's
cores (worker processes over the independent (batch, head) pairs).
"""
import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}    # dense matrix-core peaks per input type


def algorithmic_bytes(B, T, H, dk, dv, es, rank=0):
    """Bytes the layer must move: read q, k, g, bx, v, w (+ U_b factors), write o,
    the fp32 final state and the fp32 final mean."""
    per_tok = (4 * dk + dv + 1 + dv) * es
    return B * T * H * per_tok + H * rank * (dk + dv) * es + B * H * dv * dk * 4 + B * H * dv * 4


def algorithmic_flops(B, T, H, dk, dv, L, rank=0):
    """FLOPs of the triangle-aware WY chunk form (2 per multiply-add), per chunk
    of L tokens: the gated Grams A and P (L(L-1)/2 d_k each), the unit-lower
    inverse (L(L-1)(L-2)/6), W and U (L(L+1)/2 (d_k + d_v)), the residual, the
    state update and the inter-chunk readout (3 L d_k d_v), the masked
    intra-chunk readout (L(L-1)/2 d_v), the content bias and the chunk mean
    (r (d_k + d_v) + L d_v). Work an implementation adds on top (the affine maps
    of the two-pass split) is not counted."""
    def chunk(l):
        mac = (l * (l - 1) * dk + l * (l - 1) * (l - 2) // 6 + l * (l + 1) // 2 * (dk + dv)
               + 3 * l * dk * dv + l * (l - 1) // 2 * dv + rank * (dk + dv) + l * dv)
        return 2 * mac
    full, tail = divmod(T, L)
    return B * H * (full * chunk(L) + (chunk(tail) if tail else 0))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_workers():
    """Worker processes for the oracle baseline: the CPUs this process may run
    on, at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_task(args):
    """One worker's share of the oracle baseline (runs in a spawned process
    with BLAS limited to one thread): `passes` runs of the float64 oracle over
    a group of (batch, head) pairs. Returns the wall-clock start and end."""
    from threadpoolctl import threadpool_limits
    from oracle import carve_forward
    x, L, ub, passes = args
    with threadpool_limits(1):
        t0 = time.time()
        for _ in range(passes):
            carve_forward(*x, L, **ub)
        return t0, time.time()


def cpu_baseline(wl, inp, budget_s):
    """Time the float64 oracle on this host's cores, on a bounded sample of the
    workload. The (batch, head) pairs are independent, so they are split into
    one group per worker process (BLAS at one thread each) and the groups run
    in parallel; the sample is whole sequences when the work fits the budget,
    else a prefix of every sequence sized to it. Returns the head-token rate in
    tokens/s (batch rows x time steps, all heads), as the GPU value is, over
    the wall time of the parallel passes."""
    import multiprocessing as mp
    import numpy as np
    from chunk_gated_delta_carve_amd.workloads import to_f64

    nw = oracle_workers()
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    groups = [pairs[i::nw] for i in range(nw) if pairs[i::nw]]

    def tasks(Tp):
        out = []
        for grp in groups:
            x = [np.ascontiguousarray(to_f64(np.stack([inp[k][b, :Tp, h] for b, h in grp], axis=1)[None], wl.dtype))
                 for k in ("q", "k", "v", "g", "bx", "w")]
            ub = {}
            if wl.rank > 0:
                hs = [h for _, h in grp]
                ub = dict(U_down=to_f64(inp["U_down"][hs], wl.dtype), U_up=to_f64(inp["U_up"][hs], wl.dtype))
            out.append((x, wl.L, ub))
        return out

    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = "1"                            # inherited by the spawned workers
    try:
        with mp.get_context("spawn").Pool(len(groups)) as pool:
            def run(Tp, passes):
                spans = pool.map(_oracle_task, [t + (passes,) for t in tasks(Tp)])
                return max(e for _, e in spans) - min(b for b, _ in spans)
            run(min(wl.T, wl.L), 1)                           # start-up and imports, untimed
            probe_T = min(wl.T, 2 * wl.L)
            rate = probe_T / run(probe_T, 1)                  # time steps per second, all pairs
            Tp = wl.T if wl.T / rate <= budget_s else max(wl.L, int(budget_s * rate) // wl.L * wl.L)
            per = max(1, int(budget_s * rate / Tp))
            wall, passes = 0.0, 0
            while wall < budget_s:
                wall += run(Tp, per)
                passes += per
            steps = Tp * passes
    finally:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    what = ("the whole workload" if Tp == wl.T else f"the first {Tp} of {wl.T} time steps")
    return {"value": wl.B * steps / wall, "unit": "tokens/s", "cores": len(groups), "kind": "oracle",
            "sample": f"{what} (B={wl.B}, all {wl.H} heads), {passes} pass(es), {wall:.1f} s wall; "
                      f"{len(groups)} worker processes over the (batch, head) pairs, one BLAS thread each, "
                      f"on {cpu_model()}"}


KERNEL_SOURCES = ("chunk_gated_delta_carve_amd/csrc/carve_lib.hip",
                  "chunk_gated_delta_carve_amd/csrc/kernels/common.h",
                  "chunk_gated_delta_carve_amd/csrc/kernels/block.h",
                  "chunk_gated_delta_carve_amd/csrc/kernels/kernels.h")
COPY_BYTES = 256 * 1024 * 1024      # calibration copy: reads and writes this many bytes


def sources_sha():
    """Hash of the kernel sources with comments and blank lines removed, so a
    comment edit does not retire the counter summary."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for ln in text.splitlines():
            code = ln.split("//", 1)[0].rstrip()
            if code.strip():
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_file(wl):
    return os.path.join(ROOT, "profiles", f"carve_chunk_fwd_{wl.tag()}_hbm_traffic.md")


def measured_traffic(wl):
    """HBM bytes per launch from the committed rocprofv3 counter summary for this
    workload, or None when there is none or the kernel sources have changed
    since the counters were taken."""
    path = traffic_file(wl)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for ln in f:
            if ln.startswith("- ") and ": " in ln:
                key, val = ln[2:].split(": ", 1)
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel sources sha256/16") != sources_sha():
        return None
    return float(fields["HBM bytes per launch"])


def write_traffic_summary(wl, fetch_csv, write_csv, commands):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; csv output)
    over `bench.py --calibrate-copy` into the summary that measured_traffic reads.
    Each counter is scaled by what it reads for a plain copy of COPY_BYTES."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        vals = defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals[r["Kernel_Name"]].append(float(r["Counter_Value"]) * 1024.0)   # KiB -> bytes
        return vals

    def copy_kernel(vals):
        # the calibration copy is the only negation kernel in the process
        cands = [(k, v) for k, v in vals.items() if "neg" in k.lower() and min(v) > 0.5 * COPY_BYTES]
        if not cands:
            raise SystemExit("no calibration copy kernel found in " + str(list(vals)))
        return cands[0]

    rows, scaled = [], 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        cname, cv = copy_kernel(vals)
        factor = (sum(cv) / len(cv)) / COPY_BYTES
        for name, v in sorted(vals.items()):
            if not name.startswith("void carve::") and "carve_" not in name:
                continue
            avg = sum(v) / len(v)
            scaled += avg / factor
            rows.append((counter, _demangle([name])[0], len(v), avg, factor, avg / factor))
        rows.append((counter, "calibration: " + cname.split("(")[0][:60], len(cv), sum(cv) / len(cv), factor,
                     COPY_BYTES))
    with open(traffic_file(wl), "w") as f:
        f.write(f"# HBM traffic of carve_chunk_fwd, {wl.describe()}\n\n")
        f.write("Counters from two rocprofv3 runs over the same committed command, one counter each:\n\n")
        for c in commands:
            f.write(f"    {c}\n")
        f.write("\nEach per-dispatch value (KiB) is divided by the factor that the same counter reads for a "
                f"plain device copy of {COPY_BYTES} bytes (read once, written once), run in the same process.\n\n")
        f.write("| counter | kernel | dispatches | bytes per dispatch (raw) | copy factor | bytes (scaled) |\n")
        f.write("|---|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| {r[0]} | `{r[1]}` | {r[2]} | {r[3]:.0f} | {r[4]:.4f} | {r[5]:.0f} |\n")
        f.write(f"\n- HBM bytes per launch: {scaled:.0f}\n")
        f.write(f"- algorithmic bytes per launch: {algorithmic_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv, 2 if wl.dtype == 'bf16' else 4, wl.rank)}\n")
        f.write(f"- kernel sources sha256/16: `{sources_sha()}`\n")
    print(open(traffic_file(wl)).read())


def mfma_file(wl):
    return os.path.join(ROOT, "profiles", f"carve_chunk_fwd_{wl.tag()}_mfma.md")


def measured_mfma(wl):
    """Matrix-core counters per call from the committed rocprofv3 summary for this
    workload ({"mfma_flops": executed MFMA FLOPs, "mfma_busy": busy fraction of
    the SIMDs' matrix cores over the kernels' active time}), or None when there is
    none or the kernel sources have changed since the counters were taken."""
    path = mfma_file(wl)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for ln in f:
            if ln.startswith("- ") and ": " in ln:
                key, val = ln[2:].split(": ", 1)
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel sources sha256/16") != sources_sha():
        return None
    return {"mfma_flops": float(fields["executed MFMA FLOPs per launch"]),
            "mfma_busy": float(fields["MFMA busy fraction (time-weighted)"])}


def write_mfma_summary(wl, pmc_csv, trace_csv, commands):
    """Turn a rocprofv3 --pmc run (MfmaUtil, MfmaFlopsBF16 and MfmaFlopsF32; csv)
    and a --kernel-trace --stats run (for the kernels' durations) over bench.py
    into the summary that measured_mfma reads."""
    import csv
    from collections import defaultdict

    vals = defaultdict(lambda: defaultdict(list))
    with open(pmc_csv) as f:
        for r in csv.DictReader(f):
            if "carve_" in r["Kernel_Name"]:
                vals[_demangle([r["Kernel_Name"]])[0]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    dur = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            if "carve_" in r["Name"]:
                dur[_demangle([r["Name"]])[0]] = float(r["MinNs"]) * 1e-9
    rows, flops_tot, busy_w, t_tot = [], 0.0, 0.0, 0.0
    for name, c in sorted(vals.items()):
        avg = {k: sum(v) / len(v) for k, v in c.items()}
        fl = avg.get("MfmaFlopsBF16", 0.0) + avg.get("MfmaFlopsF32", 0.0)
        util = avg.get("MfmaUtil", 0.0) / 100.0
        t = dur.get(name)
        rows.append((name, len(c.get("MfmaUtil", [])), fl, util, t))
        flops_tot += fl
        if t:
            busy_w += util * t
            t_tot += t
    alg = algorithmic_flops(wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.L, wl.rank)
    peak = MFMA_PEAK_TFLOPS["bf16" if wl.dtype == "bf16" else "f32"]
    with open(mfma_file(wl), "w") as f:
        f.write(f"# Matrix-core use of carve_chunk_fwd, {wl.describe()}\n\n")
        f.write("Counters from one rocprofv3 --pmc run (derived metrics MfmaUtil = busy cycles of the "
                "SIMDs' matrix cores over GRBM_GUI_ACTIVE x SIMD count, MfmaFlopsBF16/F32 = MFMA "
                "operations x 512), durations (fastest call) from one --kernel-trace --stats run of the "
                "same command:\n\n")
        for cmd in commands:
            f.write(f"    {cmd}\n")
        f.write("\n| kernel | dispatches | executed MFMA FLOPs per dispatch | MFMA busy | duration (us) | "
                "executed TFLOP/s | fraction of peak |\n|---|---|---|---|---|---|---|\n")
        for name, n, fl, util, t in rows:
            rate = fl / t / 1e12 if t else float("nan")
            f.write(f"| `{name}` | {n} | {fl:.4g} | {100 * util:.1f}% | "
                    f"{(t or float('nan')) * 1e6:.2f} | {rate:.1f} | {rate / peak:.4f} |\n")
        f.write(f"\nPeak: {peak} TFLOP/s dense ({wl.dtype} inputs). The algorithmic count of the method "
                "(triangle-aware WY chunk form, what bench.py reports as mfma.achieved) is below the "
                "executed count: the kernels form each block's affine maps (M, C, Q_eff, O_loc) as extra products, "
                "and the diagonal inverses as products of powers.\n\n")
        f.write(f"- executed MFMA FLOPs per launch: {flops_tot:.0f}\n")
        f.write(f"- algorithmic FLOPs per launch: {alg}\n")
        f.write(f"- MFMA busy fraction (time-weighted): {busy_w / t_tot if t_tot else 0.0:.4f}\n")
        f.write(f"- kernel sources sha256/16: `{sources_sha()}`\n")
    print(open(mfma_file(wl)).read())


def trace_file(wl, backward=False):
    kind = "bwd" if backward else "fwd"
    return os.path.join(ROOT, "profiles", f"carve_chunk_{kind}_{wl.tag()}_kernel_trace.md")


def _demangle(names):
    """Readable names of this library's kernels (carve::<kernel><template
    arguments>: bf16 or float, integers, booleans); other names shortened."""
    import re
    out = []
    for n in names:
        m = re.match(r"_ZN5carve(\d+)(\w+?)I(.*)EEv", n)
        if m and len(m.group(2)) >= int(m.group(1)):
            kname = m.group(2)[:int(m.group(1))]
            rest = m.group(2)[int(m.group(1)):] + "I" + m.group(3)
            args = re.findall(r"DF16b|Lb[01]E|Li\d+E|(?<![A-Za-z])f", rest.split("I", 1)[1])
            conv = {"DF16b": "bf16", "f": "float", "Lb0E": "false", "Lb1E": "true"}
            out.append(f"{kname}<" + ",".join(conv.get(x, x[2:-1]) for x in args) + ">")
        else:
            n = n.split("(")[0]
            out.append(n if len(n) <= 90 else n[:87] + "...")
    return out


def write_trace_summary(wl, stats_csv, bench_log, commands, backward=False):
    """Turn a rocprofv3 --kernel-trace --stats run (csv) over bench.py, and the
    JSON line of the same command run without the profiler, into a short
    per-kernel summary for this workload."""
    import csv
    import json
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    names = _demangle([r["Name"] for r in rows])
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    line = None
    with open(bench_log) as f:
        for ln in f:
            if ln.startswith("{"):
                line = json.loads(ln)
    path = trace_file(wl, backward)
    with open(path, "w") as f:
        f.write(f"# Kernel trace: carve_chunk_{'bwd' if backward else 'fwd'}, {wl.describe()}\n\n")
        f.write("Commands (run from the repository root on one MI355X; the first without the profiler):\n\n")
        for c in commands:
            f.write(f"    {c}\n")
        if backward:
            f.write("\nPer-kernel statistics of the profiled run (`run_kernel_stats.csv`). Every call of "
                    "carve_chunk_bwd launches each of its kernels once, the state pass twice when it both "
                    "forms the chunk-start states and runs the state-gradient chain (warm-up and timed "
                    "calls):\n\n")
        else:
            f.write("\nPer-kernel statistics of the profiled run (`run_kernel_stats.csv`). Every call of "
                    "carve_chunk_fwd launches its kernels once; bench.py makes warm-up, back-to-back, "
                    "same-input, single and cold-cache calls, so the averages mix cache states (the fill "
                    "kernel is the untimed 512 MB cache flush before each cold-cache call, the negation kernel "
                    "the device-copy reference):\n\n")
        f.write("| kernel | calls | average (us) | min (us) | max (us) | share |\n|---|---|---|---|---|---|\n")
        for r, n in zip(rows, names):
            f.write(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                    f"{float(r['MaxNs']) / 1e3:.2f} | {100 * float(r['TotalDurationNs']) / total:.1f}% |\n")
        carve = [(r, n) for r, n in zip(rows, names) if "carve_" in r["Name"]]
        if backward and carve:
            # calls of carve_chunk_bwd: the fewest launches of any of its kernels
            ncall = min(int(r["Calls"]) for r, _ in carve)
            f.write(f"\n- CARVE kernel time per carve_chunk_bwd call ({ncall} calls): "
                    f"{sum(float(r['TotalDurationNs']) for r, _ in carve) / ncall / 1e3:.2f} us\n")
        else:
            f.write(f"\n- sum of the CARVE kernels' averages per call: "
                    f"{sum(float(r['AverageNs']) for r, _ in carve) / 1e3:.2f} us\n")
        if line:
            rf = line["roofline"]
            timing = rf.get("timing", "HIP events around the timed calls").split(",")[0]
            f.write(f"- without the profiler: {line['value']:.4g} tokens/s, `ms_per_step` {line['ms_per_step']:.4f}, "
                    f"`kernel_ms` {rf['kernel_ms']:.4f} ({timing}), HBM fraction "
                    f"{rf['frac']:.4f} of {rf['peak']:.0f} GB/s")
            mf = line.get("mfma") or {}
            if mf.get("frac") is not None:
                f.write(f", MFMA fraction {mf['frac']:.4f} (algorithmic FLOPs)")
            if "kernel_ms_same_input" in rf:
                f.write(f"; same-input {rf['kernel_ms_same_input']:.4f} ms, flushed-cache median "
                        f"{rf.get('kernel_ms_flushed_median', float('nan')):.4f} ms")
            f.write("\n")
            cb = line.get("cpu_baseline")
            if cb:
                f.write(f"- oracle on the host: {cb['value']:.4g} {cb['unit']} ({cb['cores']} workers; {cb['sample']})\n")
        f.write(f"- kernel sources sha256/16: `{sources_sha()}`\n")
    print(open(path).read())


def backward_bytes(B, T, H, dk, dv, es, rank=0):
    """Bytes the backward pass must move: read q, k, g, bx, v, w and d_o (+ U_b
    factors), write dq, dk, dg, dbx, dv, dw (+ the factors' fp32 gradients) and
    the fp32 gradients of the incoming state and mean."""
    reads = B * T * H * (4 * dk + 2 * dv + 1) * es + H * rank * (dk + dv) * es
    writes = B * T * H * (4 * dk + dv + 1) * es + H * rank * (dk + dv) * 4 + B * H * (dv * dk + dv) * 4
    return reads + writes


def backward_cpu_baseline(wl, inp, do, budget_s):
    """The float64 oracle's backward pass, single-threaded, on a prefix of every
    sequence sized to the budget (at most 256 time steps: the oracle keeps every
    token's state). Returns tokens/s as the GPU value is."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import carve_backward
    from chunk_gated_delta_carve_amd.workloads import to_f64

    def run(Tp):
        f = lambda x: np.ascontiguousarray(to_f64(x[:, :Tp], wl.dtype))
        ub = {}
        if wl.rank > 0:
            ub = dict(U_down=to_f64(inp["U_down"], wl.dtype), U_up=to_f64(inp["U_up"], wl.dtype))
        t0 = time.perf_counter()
        carve_backward(*(f(inp[k]) for k in ("q", "k", "v", "g", "bx", "w")), wl.L, f(do), **ub)
        return time.perf_counter() - t0

    with threadpool_limits(1):
        probe_T = min(wl.T, wl.L)
        rate = probe_T / run(probe_T)
        Tp = min(wl.T, 256, max(wl.L, int(budget_s * rate) // wl.L * wl.L))
        spent, steps, passes = 0.0, 0, 0
        while spent < budget_s:
            spent += run(Tp)
            steps += Tp
            passes += 1
    return {"value": wl.B * steps / spent, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {Tp} of {wl.T} time steps (B={wl.B}, all {wl.H} heads), {passes} pass(es), "
                      f"{spent:.1f} s, one thread"}


def backward_kernels(wl, rank):
    """The kernels one carve_chunk_bwd call launches on this workload."""
    if rank == 0 and wl.dtype == "bf16" and wl.dk == 64:
        return ("carve_intra_kernel + carve_state_kernel (64-token block start states) + carve_bwd_image_kernel + "
                "carve_state_kernel (state-gradient chain) + carve_bwd_chunk_kernel (one call)")
    if rank == 0:
        pre = ("carve_intra_kernel + carve_state_kernel (chunk-start states) + "
               if wl.dtype == "bf16" and wl.L % 64 == 0 else "")
        return pre + "carve_bwd_split_kernel + carve_bwd_finish_kernel (one call)"
    if wl.dk == 64 and wl.dtype == "bf16" and wl.L == 64:
        return ("carve_chunk_serial_kernel (chunk-start states, gate biases and means) + "
                "carve_bwd_chunk_serial_kernel + carve_bwd_ub_kernel (one call)")
    if wl.dk == 64:
        return "carve_bwd_split_kernel + carve_bwd_finish_kernel + carve_bwd_ub_kernel (one call)"
    return "carve_bwd_kernel + carve_bwd_ub_kernel (one call)"


def bench_backward(args, wl):
    """carve_chunk_bwd on the workload, from seeded output gradients d_o (no
    state or mean gradients, as in a training step that starts from zeros):
    K back-to-back calls between two HIP events on the launch stream."""
    import numpy as np
    import torch

    from chunk_gated_delta_carve_amd import chunk_bwd
    from chunk_gated_delta_carve_amd.workloads import bf16_bits_from_f32, make_inputs, to_torch

    inp = make_inputs(wl, decay_logits=args.decay_logits)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    B, T, H, dk, dv, L, rank = wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.L, wl.rank
    do = np.random.default_rng(wl.seed + 17).standard_normal((B, T, H, dv)).astype(np.float32)
    do = do if wl.dtype == "f32" else bf16_bits_from_f32(do)
    d_o = to_torch(do, wl.dtype)
    ub = (t["U_down"], t["U_up"]) if rank else (None, None)
    from chunk_gated_delta_carve_amd import recurrent_ref_shapes
    tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    ws = torch.empty(int(recurrent_ref_shapes(B, H, T, dk, dv, L, rank, tdtype, qk_l2norm=args.qk_l2norm)
                         .bwd_workspace_bytes), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    out = None

    def step():
        nonlocal out
        out = chunk_bwd(*(t[k] for k in ("q", "k", "v", "g", "bx", "w")), d_o, L=L, ub_down=ub[0], ub_up=ub[1],
                        decay_logits=args.decay_logits, qk_l2norm=args.qk_l2norm, workspace=ws, out=out)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    ev_start, ev_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev_start.record(stream)
    for _ in range(args.steps):
        step()
    ev_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    kernel_ms = ev_start.elapsed_time(ev_end) / args.steps
    es = 2 if wl.dtype == "bf16" else 4
    alg = backward_bytes(B, T, H, dk, dv, es, rank)
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    line = {
        "metric": f"tokens/s of carve_chunk_bwd (backward), B{B} H{H} T{T} d{dk} L{L} {wl.dtype}",
        "value": B * T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; inputs as for carve_chunk_fwd, d_o N(0,1))",
        "config": {"workload": f"carve_chunk_bwd B{B} H{H} T{T} dk{dk} dv{dv} L{L} {wl.dtype}, "
                               + (f"content projection rank {rank}" if rank else "no content projection"),
                   "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "L": L, "rank": rank,
                   "decay_input": "raw logits, -softplus in-kernel" if args.decay_logits else "log-decay g",
                   "qk": "L2-normalised in-kernel" if args.qk_l2norm else "as given"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": backward_kernels(wl, rank),
                     "kernel_ms": kernel_ms, "algorithmic_bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline and not args.decay_logits and not args.qk_l2norm:
        line["cpu_baseline"] = backward_cpu_baseline(wl, inp, do, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def decode_bytes(B, H, dk, dv, es, rank=0):
    """Bytes one decode step must move: read the token's q, k, g, b_x, v, w and
    the U_b factors, read and write the fp32 state, mean and chunk sum, write o."""
    return (B * H * ((4 * dk + dv + 1) * es + dv * es) + H * rank * (dk + dv) * es
            + 2 * B * H * (dv * dk + 2 * dv) * 4)


def decode_cpu_baseline(wl, inp, budget_s):
    """The float64 oracle's decode step, single-threaded, on a bounded number of
    steps of the same workload. Returns tokens/s (batch rows per second)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import carve_step
    from chunk_gated_delta_carve_amd.workloads import to_f64

    f = lambda key: to_f64(inp[key], wl.dtype)
    x = {key: f(key) for key in ("q", "k", "v", "g", "bx", "w")}
    Ud, Uu = (f("U_down"), f("U_up")) if wl.rank else (None, None)
    S = np.zeros((wl.B, wl.H, wl.dv, wl.dk))
    m = np.zeros((wl.B, wl.H, wl.dv))
    acc = np.zeros_like(m)
    steps, spent = 0, 0.0
    with threadpool_limits(1):
        while spent < budget_s:
            s = steps % wl.T
            t0 = time.perf_counter()
            _, S, m, acc = carve_step(S, m, acc, s % wl.L, *(x[key][:, s] for key in ("q", "k", "v", "g", "bx", "w")),
                                      wl.L, Ud, Uu)
            spent += time.perf_counter() - t0
            steps += 1
    return {"value": wl.B * steps / spent, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} decode steps of the workload (B={wl.B}, all {wl.H} heads), {spent:.1f} s, one thread"}


def bench_decode(args, wl):
    """Decode steps (carve_recurrent_step), each one token of every (batch,
    head), cycling through the workload's T tokens with pos = step mod L. A
    serving loop launches them from a HIP graph: one chunk of L steps is
    captured once and replayed, so the timed region is whole replays (the
    step count rounds up to a multiple of L). The same steps launched one call
    at a time from Python are timed as well (`kernel_ms_eager`): there the
    per-call host work, not the GPU, sets the pace."""
    import numpy as np
    import torch

    from chunk_gated_delta_carve_amd.api import recurrent_step
    from chunk_gated_delta_carve_amd.workloads import make_inputs, to_torch

    logits = args.decay_logits
    inp = make_inputs(wl, decay_logits=logits)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    toks = [{k: t[k][:, s].clone() for k in ("q", "k", "v", "g", "bx", "w")} for s in range(wl.T)]
    ub = (t["U_down"], t["U_up"]) if wl.rank else (None, None)
    B, H, dk, dv, L = wl.B, wl.H, wl.dk, wl.dv, wl.L
    S = torch.zeros((B, H, dv, dk), dtype=torch.float32, device="cuda")
    m = torch.zeros((B, H, dv), dtype=torch.float32, device="cuda")
    acc = torch.zeros_like(m)
    o = torch.empty((B, H, dv), dtype=toks[0]["q"].dtype, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        x = toks[i % wl.T]
        recurrent_step(x["q"], x["k"], x["v"], x["g"], x["bx"], x["w"], S, m, acc, i % L, L, *ub, out=o,
                       decay_logits=logits)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev_start, ev_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev_end.record(stream)
    torch.cuda.synchronize()
    kernel_ms_eager = ev_start.elapsed_time(ev_end) / args.steps

    # one chunk of steps (positions 0 .. L-1) in a graph
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(L):
                step(i)
    stream.wait_stream(side)
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, (args.steps + L - 1) // L)
    t0 = time.perf_counter()
    ev_start.record(stream)
    for _ in range(reps):
        graph.replay()
    ev_end.record(stream)
    torch.cuda.synchronize()
    steps = reps * L
    ms_per_step = 1e3 * (time.perf_counter() - t0) / steps
    kernel_ms = ev_start.elapsed_time(ev_end) / steps
    es = 2 if wl.dtype == "bf16" else 4
    alg = decode_bytes(B, H, dk, dv, es, wl.rank)
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    line = {
        "metric": "tokens/s of carve_recurrent_step (decode), one token per (batch, head) per step",
        "value": B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; distributions as for carve_chunk_fwd)",
        "config": {"workload": f"carve_recurrent_step B{B} H{H} dk{dk} dv{dv} L{L} {wl.dtype}, "
                               + (f"content projection rank {wl.rank}" if wl.rank else "no content projection"),
                   "B": B, "H": H, "dk": dk, "dv": dv, "L": L, "rank": wl.rank,
                   "decay_input": "raw logits, -softplus in-kernel" if logits else "log-decay g"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "carve_step_kernel",
                     "kernel_ms": kernel_ms, "algorithmic_bytes_per_launch": alg,
                     "kernel_ms_eager": kernel_ms_eager},
    }
    if not args.no_cpu_baseline and not logits:
        line["cpu_baseline"] = decode_cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="init_equiv",
                    help="workload to time (default: the B4 H12 T2048 d64 L64 bf16 shape; "
                         "`decode` times the one-token step instead)")
    ap.add_argument("--L", type=int, default=None, help="override the chunk length")
    ap.add_argument("--decay-logits", action="store_true",
                    help="pass raw decay logits and let the kernels form g = -softplus(.) (CARVE_DECAY_LOGITS); "
                         "also times the unfused alternative (a torch softplus pass, then the plain call)")
    ap.add_argument("--input-copies", type=int, default=4,
                    help="input copies the timed steps rotate through, so that no step finds its inputs in "
                         "the 256 MB Infinity Cache (1: every step reads the same inputs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU work budget of the oracle baseline sample")
    ap.add_argument("--qk-l2norm", action="store_true",
                    help="let the kernels normalise q and k per token (CARVE_QK_L2NORM); also times the unfused "
                         "alternative (torch normalises q and k, then the plain call)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass carve_chunk_bwd on the workload instead of the forward")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain device copy of known size first (for counter calibration)")
    ap.add_argument("--write-traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc csv files and exit")
    ap.add_argument("--write-mfma-summary", nargs=2, metavar=("PMC_CSV", "STATS_CSV"),
                    help="write the matrix-core summary from a rocprofv3 --pmc csv (MfmaUtil, MfmaFlopsBF16, "
                         "MfmaFlopsF32) and a --kernel-trace --stats csv, and exit")
    ap.add_argument("--write-trace-summary", nargs=2, metavar=("STATS_CSV", "BENCH_LOG"),
                    help="write the kernel-trace summary from a rocprofv3 --kernel-trace --stats csv and the log "
                         "of the same command run without the profiler, and exit")
    ap.add_argument("--commands", nargs="*", default=[], help="commands recorded in a counter summary")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(every (batch, head) pair is independent, so sharding is data placement)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from chunk_gated_delta_carve_amd import chunk_fwd
    from chunk_gated_delta_carve_amd.workloads import WORKLOADS, make_inputs, to_f64, to_torch

    wl = WORKLOADS[args.workload]
    if args.L is not None:
        wl = wl.with_(L=args.L)
    if args.write_traffic_summary:
        write_traffic_summary(wl, *args.write_traffic_summary, args.commands)
        return
    if args.write_mfma_summary:
        write_mfma_summary(wl, *args.write_mfma_summary, args.commands)
        return
    if args.write_trace_summary:
        write_trace_summary(wl, *args.write_trace_summary, args.commands, backward=args.backward)
        return
    if args.workload == "decode":
        bench_decode(args, wl)
        return
    if args.backward:
        bench_backward(args, wl)
        return
    logits, norm = args.decay_logits, args.qk_l2norm
    special = logits or norm                           # an input mode other than the profiled one
    inp = make_inputs(wl, decay_logits=logits)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    B, T, H, dk, dv, L, rank = wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.L, wl.rank
    tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    es = 2 if wl.dtype == "bf16" else 4
    o = torch.empty((B, T, H, dv), dtype=tdtype, device="cuda")
    stream = torch.cuda.current_stream()
    from chunk_gated_delta_carve_amd import recurrent_ref_shapes
    ws_bytes = int(recurrent_ref_shapes(B, H, T, dk, dv, L, rank, tdtype).workspace_bytes)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    ub = (t["U_down"], t["U_up"]) if rank > 0 else (None, None)

    # Input copies that the timed steps rotate through: a copy is read again
    # only after the other copies' steps have streamed far more than the 256
    # MB Infinity Cache, so every timed step reads its inputs from HBM.
    copies = [t] + [{k: v.clone() for k, v in t.items()} for _ in range(max(1, args.input_copies) - 1)]
    rot = [0]

    def step(x=None):
        if x is None:
            x = copies[rot[0] % len(copies)]
            rot[0] += 1
        return chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["bx"], x["w"], L=L, ub_down=ub[0], ub_up=ub[1],
                         return_state=True, out=o, workspace=ws, decay_logits=logits, qk_l2norm=norm)

    g_buf = torch.empty_like(t["g"])

    def unfused_step():
        # what a caller without the fused input handling runs: materialise g
        # and/or the normalised q and k, then the plain call
        g = t["g"]
        if logits:
            torch.neg(torch.nn.functional.softplus(t["g"]), out=g_buf)
            g = g_buf
        q, k = t["q"], t["k"]
        if norm:
            q = torch.nn.functional.normalize(q, dim=-1, eps=1e-12)
            k = torch.nn.functional.normalize(k, dim=-1, eps=1e-12)
        return chunk_fwd(q, k, t["v"], g, t["bx"], t["w"], L=L, ub_down=ub[0], ub_up=ub[1],
                         return_state=True, out=o, workspace=ws)

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)                    # one elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K back-to-back steps, rotating through the input copies,
    # between two HIP events on the launch stream (no events between the steps,
    # so nothing but the steps runs there)
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_start.record(stream)
    for _ in range(args.steps):
        step()
    ev_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    avg_kernel_ms = ev_start.elapsed_time(ev_end) / args.steps   # GPU time of one call

    # the same, every step on one input copy (its inputs stay in the caches)
    s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_.record(stream)
    for _ in range(args.steps):
        step(copies[0])
    e_.record(stream)
    torch.cuda.synchronize()
    same_input_ms = s_.elapsed_time(e_) / args.steps

    # single calls, each between its own pair of events: median and minimum
    single = []
    for _ in range(20):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        step()
        e.record(stream)
        torch.cuda.synchronize()
        single.append(s.elapsed_time(e))

    # reference: what a plain device copy (one elementwise kernel that reads and
    # writes COPY_BYTES) reaches on this GPU
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(10):
        torch.neg(src, out=dst)
    e.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_BYTES * 10 / (s.elapsed_time(e) * 1e-3) / 1e9
    del src, dst

    # single calls with every cache flushed before each (a 512 MB write, untimed)
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    cold = []
    for _ in range(10):
        flush.fill_(1.0)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        step()
        e.record(stream)
        torch.cuda.synchronize()
        cold.append(s.elapsed_time(e))
    del flush

    unfused_ms = None
    if special:
        for _ in range(3):
            unfused_step()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(args.steps):
            unfused_step()
        e.record(stream)
        torch.cuda.synchronize()
        unfused_ms = s.elapsed_time(e) / args.steps

    alg = algorithmic_bytes(B, T, H, dk, dv, es, rank)
    achieved = alg / (avg_kernel_ms * 1e-3) / 1e9
    flops = algorithmic_flops(B, T, H, dk, dv, L, rank)
    tflops = flops / (avg_kernel_ms * 1e-3) / 1e12
    mfma_peak = MFMA_PEAK_TFLOPS["bf16" if wl.dtype == "bf16" else "f32"]
    tokens = B * T
    parallel = rank == 0 and wl.dtype == "bf16"
    kernels = ("carve_intra_kernel + carve_state_kernel (one call)" if parallel
               else "carve_chunk_serial_kernel")
    workload = (f"carve_chunk_fwd B{B} H{H} T{T} dk{dk} dv{dv} L{L} {wl.dtype}, "
                + ("no content projection" if rank == 0 else f"content projection rank {rank}"))
    line = {
        "metric": "tokens/s + MFMA/HBM roofline % of carve_chunk_fwd, B4 H12 T2048 d64 L64 bf16",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), "
                + ("g = raw decay logits N(0,1), activated in-kernel" if logits else "g=-softplus(N(0,1))")
                + ", bx N(0,1), w=sigmoid(N(0,1))" + (f", U_b factors N(0,{wl.ub_std})" if rank else "") + ")",
        "config": {"workload": workload, "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "L": L, "rank": rank,
                   "decay_input": "raw logits, -softplus in-kernel" if logits else "log-decay g",
                   "qk": "normalised in-kernel" if norm else "used as given"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     # the committed counter summaries are of the plain launch
                     "traffic": None if special else measured_traffic(wl),
                     "kernel": kernels, "kernel_ms": avg_kernel_ms,
                     "timing": f"HIP events around {args.steps} back-to-back calls that rotate through "
                               f"{len(copies)} copies of the inputs (each copy's inputs are out of the "
                               "caches when it is read again)",
                     "algorithmic_bytes_per_launch": alg,
                     "kernel_ms_same_input": same_input_ms,
                     "kernel_ms_flushed_median": float(np.median(cold)),
                     "kernel_ms_single_median": float(np.median(single)),
                     "kernel_ms_single_min": float(np.min(single)), "copy_kernel_gbs": copy_gbs},
        # the matrix-core roofline of the same call: not the bound (the path's
        # FLOP per byte is far below the MFMA/HBM ridge), reported beside it
        "mfma": {"achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s", "frac": tflops / mfma_peak,
                 "algorithmic_flops_per_launch": flops, "counters": None if special else measured_mfma(wl)},
    }
    if special:
        line["unfused"] = {"kernel_ms": unfused_ms, "what": "torch forms " + " and ".join(
            (["-softplus(a) into a g tensor"] if logits else []) + (["normalised q and k"] if norm else []))
            + ", then the plain call (the round trip through HBM that the fused form avoids)"}
    if not args.no_cpu_baseline and not special:
        line["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
