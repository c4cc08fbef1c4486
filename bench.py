"""Benchmark of carve_chunk_fwd on one MI355X.

One step = one forward pass of the CARVE layer over the batch (every stage of
the path: gate prep, gated Grams and triangular inverse, W/U, the serial state
pass, output and chunk mean), writing o, the final state and the final mean.
Workload: B=4, H=12, T=2048, d_k=d_v=64, L=64, bf16 inputs with fp32
accumulation, no content projection (seeded synthetic data).

Prints one JSON line. `roofline` covers the dominant kernel: algorithmic bytes
per launch over its average duration, timed with HIP events on the stream the
kernel runs on. `cpu_baseline` is the float64 oracle timed on this host.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(B, T, H, dk, dv, es, rank=0):
    """Bytes the layer must move: read q, k, g, bx, v, w (+ U_b factors), write o,
    the fp32 final state and the fp32 final mean."""
    per_tok = (4 * dk + dv + 1 + dv) * es
    return B * T * H * per_tok + H * rank * (dk + dv) * es + B * H * dv * dk * 4 + B * H * dv * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (batch, head) pair is independent, so sharding is data placement)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from chunk_gated_delta_carve_amd import chunk_fwd
    from chunk_gated_delta_carve_amd.workloads import WORKLOADS, make_inputs, to_f64, to_torch

    wl = WORKLOADS["init_equiv"]
    inp = make_inputs(wl)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    B, T, H, dk, dv, L = wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.L
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    from chunk_gated_delta_carve_amd import recurrent_ref_shapes
    ws_bytes = int(recurrent_ref_shapes(B, H, T, dk, dv, L, 0, torch.bfloat16).workspace_bytes)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def step():
        return chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["bx"], t["w"], L=L, return_state=True, out=o,
                         workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K back-to-back steps; per-launch HIP events on the same stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = 1e3 * wall / args.steps
    avg_kernel_ms = float(np.mean(kernel_ms))

    # the same launch with the caches flushed before it (512 MB write, untimed)
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

    alg = algorithmic_bytes(B, T, H, dk, dv, 2)
    achieved = alg / (avg_kernel_ms * 1e-3) / 1e9
    tokens = B * T
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
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), g=-softplus(N(0,1)), bx N(0,1), w=sigmoid(N(0,1)))",
        "config": {"workload": "carve_chunk_fwd B4 H12 T2048 dk64 dv64 L64 bf16, no content projection",
                   "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "L": L, "rank": 0},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "carve_intra_kernel + carve_state_kernel (one call)", "kernel_ms": avg_kernel_ms,
                     "algorithmic_bytes_per_launch": alg, "kernel_ms_cold_cache": float(np.median(cold))},
    }
    if not args.no_cpu_baseline:
        from oracle import carve_forward
        f = lambda k: to_f64(inp[k], wl.dtype)
        tb = time.perf_counter()
        carve_forward(f("q"), f("k"), f("v"), f("g"), f("bx"), f("w"), L)
        cpu_s = time.perf_counter() - tb
        line["cpu_baseline"] = {"value": tokens / cpu_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                "sample": f"the whole workload (B={B}, T={T}, all {H} heads), one process, "
                                          f"{cpu_s:.1f} s"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
