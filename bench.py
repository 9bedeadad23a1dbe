"""Benchmark of dust_estimate on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole dust_estimate call (every stage: base GEMM, noise +
loss change, centring and credit, reweighting, outer product) over one batch
of synthetic inputs already resident in HBM; for the local-scoring workloads
(kv_local_bf16, q_local_bf16) one dust_estimate_local call, and for the
cross-entropy head (head_ce_bf16) one dust_estimate_head call, whose rows
are counted per 256-column slab (K*T*V/256), and for the token embedding
(embed_bf16) one dust_estimate_embedding call (gather, estimator, and the
reassembly of G_E divided by the token count).  The default workload is the
"bf16 layer" (T = 4096 tokens in 8 sequences of 512, d_in = d_out = 512,
K = 64 antithetic draws, sigma = 1e-2, gamma = 0).  Prints one JSON line:
draw-token-rows per second (K*T per step; K*T*V/256 for the head), the ALU roofline of the dominant
kernel timed with HIP events inside the timed region, and the fp64 CPU
oracle timed on a bounded sample on this machine's host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CAL_COPY_BYTES = 256 << 20
# every source the kernels and their launch configuration are built from
KERNEL_SOURCES = ["token_activation_perturbation_amd/csrc/" + f for f in (
    "dust_kernels.hip", "dust_noise.hpp", "dust_gemm.hpp", "dust_reassemble.hpp",
    "dust_plan.hpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("kernel") != kernel:
        return None
    if entry.get("source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def cpu_baseline(w, inp, budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample: whole sequences of
    the same workload (blocks of 16 tokens for the head), as many as fit the
    time budget (at least one)."""
    from oracle import oracle
    threads = min(16, oracle.default_threads())
    kw = dict(K=w.K, sigma=w.sigma, gamma=w.gamma, seed=w.noise_seed,
              antithetic=w.antithetic, seq_len=w.seq_len, threads=threads)
    # the sample is whole units: sequences, or blocks of 16 tokens for the
    # head (whose loss is per token)
    if w.head:
        unit, n_units = 16, w.T // 16
        kw = dict(K=w.K, sigma=w.sigma, seed=w.noise_seed, antithetic=w.antithetic,
                  threads=threads)

        def run(lo, hi):
            oracle.estimate_head(inp["X"], inp["W"], inp["labels"],
                                 token_range=(lo * unit, hi * unit), **kw)
    else:
        unit, n_units = w.seq_len, w.n_seq
        if w.embedding:
            def run(lo, hi):
                oracle.estimate_embedding(inp["table"], inp["ids"], inp["target"],
                                          seq_range=(lo, hi), scale=1.0 / w.T, **kw)
        elif w.local:
            def run(lo, hi):
                oracle.estimate_local(inp["X"], inp["E"], seq_range=(lo, hi), **kw)
        else:
            def run(lo, hi):
                oracle.estimate(inp["X"], inp["W"], inp["target"], seq_range=(lo, hi), **kw)
    run(0, 1)  # warm-up: the first call pays for loading and first touches
    t0 = time.perf_counter()
    run(0, 1)
    one = time.perf_counter() - t0
    n = max(1, min(n_units, int(budget_s / max(one, 1e-6))))
    # a whole workload that takes well under the budget is repeated, so the
    # figure is not a sub-second measurement (the repeats are planned from one
    # sequence's time, which overstates a whole run's: ~10 s of CPU work for
    # the default 15 s budget)
    repeats = 1
    if n == n_units:
        repeats = max(1, min(400, int(budget_s / max(one * n, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(repeats):
        run(0, n)
    elapsed = time.perf_counter() - t0
    rows = w.K * w.n_slab * unit * n * repeats
    draws = f"{w.K} draws x {w.n_slab} slabs" if w.head else f"{w.K} draws"
    what = (f"{n * unit} of {w.T} tokens ({draws}) of the benchmarked workload")
    if repeats > 1:
        what = f"the whole benchmarked workload ({w.T} tokens x {draws}) {repeats} times"
    return {"value": rows / elapsed, "unit": "draw-token-rows/s", "cores": threads,
            "kind": "oracle", "sample": f"{what}, fp64, {elapsed:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_layer",
                    help="one of the synthetic workloads of synth.py")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 to skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        sys.exit(f"bench.py: this estimator is measured on one GPU; --gpus {args.gpus} is not "
                 "supported (sharding over sequences is a design note, not built)")

    from token_activation_perturbation_amd import synth
    if args.workload not in synth.WORKLOADS:
        sys.exit(f"bench.py: unknown workload {args.workload!r}; one of "
                 f"{', '.join(synth.WORKLOAD_ORDER)}")

    import torch

    import token_activation_perturbation_amd as dust
    from token_activation_perturbation_amd import roofline

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(w)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    def to_dev(name, cast=True):
        t = torch.from_numpy(inp[name]).to(dev)
        return (t.to(tdt) if cast else t).contiguous()

    if w.embedding:
        table, tg, ids = to_dev("table"), to_dev("target"), to_dev("ids", cast=False)
    elif w.local:
        # local scoring: the draws are scored against the error estimate E
        X, E = to_dev("X"), to_dev("E", cast=False)
    elif w.head:
        X, W, labels = to_dev("X"), to_dev("W"), to_dev("labels", cast=False)
    else:
        X, W, tg = to_dev("X"), to_dev("W"), to_dev("target")
    dt_code = dust.DUST_F32 if w.dtype == "f32" else dust.DUST_BF16
    # the estimator's workspace sized for single generation where it applies
    # (gamma > 0 with antithetic pairs and enough sequence-pair chains)
    base_bytes = dust.dust_workspace_bytes(w.T, w.d_in, w.d_out, w.K, w.antithetic, dt_code)
    ws_bytes = (dust.dust_embedding_workspace_bytes(w.T, w.V, w.d_out, w.K, w.antithetic, dt_code)
                if w.embedding else base_bytes if w.head else
                dust.dust_workspace_bytes_seq(w.T, w.d_in, w.d_out, w.seq_len, w.K, w.gamma,
                                              w.antithetic, dt_code))
    chain = not w.embedding and not w.head and ws_bytes > base_bytes
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    kw = dict(K=w.K, sigma=w.sigma, gamma=w.gamma, seed=w.noise_seed, antithetic=w.antithetic,
              seq_len=w.seq_len)
    if w.head:
        kw = dict(K=w.K, sigma=w.sigma, seed=w.noise_seed, antithetic=w.antithetic)
    # an untimed plain copy of known size: rocprofv3's FETCH_SIZE / WRITE_SIZE
    # counters read on it calibrate the HBM bytes reported for our kernels
    cal_src = torch.ones(CAL_COPY_BYTES // 4, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize(dev)
    del cal_src, cal_dst

    def estimate(out):
        if w.embedding:
            return dust.dust_estimate_embedding(table, ids, tg, out=out, workspace=ws,
                                                scale=1.0 / w.T, **kw)
        if w.local:
            return dust.dust_estimate_local(X, E, out=out, workspace=ws, **kw)
        if w.head:
            return dust.dust_estimate_head(X, W, labels, out=out, workspace=ws, **kw)
        return dust.dust_estimate(X, W, tg, out=out, workspace=ws, **kw)

    out = {}
    for _ in range(args.warmup):
        out = estimate(out)
    torch.cuda.synchronize(dev)
    if not bool(torch.isfinite(out["G_E" if w.embedding else "G_W"]).all()):
        sys.exit("bench.py: non-finite weight gradient")

    # event pairs stamped by the dispatch of the dominant kernel of every
    # timed step (the library launches it with hipExtLaunchKernelGGL)
    fused = (w.gamma == 0.0 or w.seq_len == 1)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for e in starts + stops:
        e.record()  # creates the underlying hipEvent
    torch.cuda.synchronize(dev)
    dust.dust_set_timing_events(starts, stops)

    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    wall0 = time.perf_counter()
    t_begin.record()
    for _ in range(args.steps):
        estimate(out)
    t_end.record()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    dust.dust_set_timing_events([], [])
    ms_per_step = t_begin.elapsed_time(t_end) / args.steps
    kernel_ms = sum(s.elapsed_time(e) for s, e in zip(starts, stops)) / args.steps

    value = w.rows / (ms_per_step * 1e-3)
    if w.head:
        kernel = "head_ce_kernel"
        slots = roofline.head_kernel_slots(w.T, w.d_out, w.K, w.antithetic)
        min_s = roofline.head_min_seconds(w.T, w.d_out, w.K, w.antithetic)
    elif fused or chain:
        # both generate each noise value once and add P's and g's FMAs
        kernel = "fused_g0_kernel" if fused else "chain_g_kernel"
        slots = roofline.fused_kernel_slots(w.T, w.d_out, w.K, w.antithetic, local=w.local)
    else:
        kernel = "jitter_loss_kernel"
        slots = roofline.jitter_kernel_slots(w.T, w.d_out, w.K, w.antithetic, local=w.local)
    if not w.head:
        min_s = roofline.estimate_min_seconds(w.T, w.d_out, w.K, w.antithetic, local=w.local)
    achieved = slots / (kernel_ms * 1e-3) / 1e12
    peak = roofline.PEAK_SLOTS_PER_S / 1e12
    result = {
        "metric": ("slab-draw-token-rows/sec (K*T*V/256) for dust_estimate_head" if w.head else
                   "draw-token-rows/sec (K*T) for " +
                   ("dust_estimate_local" if w.local else
                    "dust_estimate_embedding" if w.embedding else "dust_estimate")),
        "value": value,
        "unit": "draw-token-rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": ("synthetic (seeded normal X and error estimate E; no dataset or trained weights)"
                 if w.local else
                 "synthetic (seeded normal X, W and uniform labels; no dataset or trained weights)"
                 if w.head else
                 "synthetic (seeded normal table and target, Zipfian token ids; no dataset or "
                 "trained weights)"
                 if w.embedding else
                 "synthetic (seeded normal X, W, target; no dataset or trained weights)"),
        "config": {**w.describe(), "input_dtype": w.dtype, "parallelism": "none (1 GPU)"},
        "roofline": {
            "bound": "alu",
            "kernel": kernel,
            "kernel_ms": kernel_ms,
            "achieved": achieved,
            "peak": peak,
            "unit": "T lane-slot/s",
            "frac": achieved / peak,
            "traffic": read_traffic(w.name, kernel),
            "end_to_end_frac": min_s / (ms_per_step * 1e-3),
        },
    }
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
