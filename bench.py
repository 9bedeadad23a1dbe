"""Benchmark of dust_estimate on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--configs all|none|NAME,NAME,...] [--cpu-budget S]

A step is one whole estimate call (every stage: base GEMM, noise + loss
change, centring and credit, reweighting, outer product) over one batch of
synthetic inputs already resident in HBM.  The headline workload (the JSON
line's top level) is the MLP up-projection (T = 16384 tokens in 32 sequences
of 512, d_in = 768, d_out = 3072, K = 256 antithetic draws, sigma = 5e-3,
gamma = 0), the largest of the estimator's five reference configurations.
The line also carries, under "configs", the same measurement for each of the
five configurations (the tiny fp32 layer, the 512-wide bf16 layer, the MLP
up-projection, the QKV projection with credit decay 0.9, the large
population of 4096 draws), and under "stages" every kernel of the headline
step against its own roofline (ALU for the noise stages, MFMA for the two
contractions, HBM for the rest), from a separate profiled pass.

Other workloads (local scoring, the cross-entropy head, the token embedding,
scores through a recomputed attention) run with --workload:
dust_estimate_local, dust_estimate_head (rows counted per 256-column slab,
K*T*V/256), dust_estimate_embedding and dust_estimate_attention calls.

The JSON line: draw-token-rows per second (K*T per step), the ALU roofline of
the dominant kernel timed with HIP events inside the timed region, the
per-stage fractions, and the fp64 CPU oracle timed on a bounded sample on
this machine's host cores (at most 16 threads: one GPU's share of the host).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CAL_COPY_BYTES = 256 << 20
# every source the kernels and their launch configuration are built from; the
# attention site's kernels are also built from ATTENTION_SOURCES, which no
# other workload's kernels use
KERNEL_SOURCES = ["token_activation_perturbation_amd/csrc/" + f for f in (
    "dust_kernels.hip", "dust_noise.hpp", "dust_gemm.hpp", "dust_reassemble.hpp",
    "dust_plan.hpp")]
ATTENTION_SOURCES = ["token_activation_perturbation_amd/csrc/dust_attention.hpp"]
# the estimator's five reference configurations, in order
REFERENCE_CONFIGS = ["tiny_f32", "bf16_layer", "mlp_up_bf16", "qkv_credit_bf16",
                     "large_population_bf16"]
HEADLINE = "mlp_up_bf16"
# host threads for the oracle: one GPU's share of the host
CPU_THREADS_MAX = 16
PROFILE_STEPS = 3


def _code_only(text: str) -> str:
    """The source without its comments and blank space, so that a change to
    a comment alone does not count as a change of the kernels."""
    token = re.compile(r'"(?:\\.|[^"\\\n])*"|/\*.*?\*/|//[^\n]*', re.S)
    text = token.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return " ".join(text.split())


def kernel_source_hash(workload: str | None = None) -> str:
    """Hash of the code (comments dropped) that the workload's kernels are
    built from: the attention sources count only for attention workloads."""
    h = hashlib.sha256()
    extra = ATTENTION_SOURCES if workload is not None and workload.startswith("attn_") else []
    for rel in KERNEL_SOURCES + extra:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
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
    if entry.get("source_hash") != kernel_source_hash(workload):
        return None
    return entry.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample: whole sequences of
    the same workload (blocks of 16 tokens for the head), as many as fit the
    time budget (at least one)."""
    from oracle import oracle
    threads = min(CPU_THREADS_MAX, oracle.default_threads())
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
    elif w.attention:
        # the oracle recomputes the attention for every draw, ~K L^2 d flops
        # per sequence and head: the sample is every sequence (one thread
        # each) with the first 2 of the K draws, whose scores do not depend
        # on the others, so rows are 2 T per run
        unit, n_units = w.seq_len, 1
        threads = min(threads, w.n_seq)
        kw = dict(K=2, sigma=w.sigma, gamma=w.gamma, seed=w.noise_seed,
                  antithetic=w.antithetic, seq_len=w.seq_len, threads=threads)

        def run(lo, hi):
            oracle.estimate_attention(inp["X"], inp["q"], inp["k"], inp["v"], inp["E"],
                                      heads=w.heads, site=w.site, **kw)
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
    if w.attention:
        rows = 2 * w.T * repeats
        what = (f"all {w.T} tokens ({w.n_seq} sequences, one thread each) x 2 of the {w.K} "
                f"draws, {repeats} time(s)")
    return {"value": rows / elapsed, "unit": "draw-token-rows/s", "cores": threads,
            "kind": "oracle", "sample": f"{what}, fp64, {elapsed:.1f} s",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "threads_note": (f"{threads} threads: the oracle's pthreads, capped at "
                             f"{CPU_THREADS_MAX} (one GPU's share of the host)")}


def dominant_kernel(w, chain: bool) -> str:
    if w.head:
        return "head_ce_kernel"
    if w.attention:
        return "attn_score_s_kernel" if w.site == "query" else "attn_score_t_kernel"
    if w.gamma == 0.0 or w.seq_len == 1:
        return "fused_g0_kernel"
    return "chain_g_kernel" if chain else "jitter_loss_kernel"


def measure(w, steps: int, warmup: int, want_inputs: bool = False):
    """Times `steps` estimate calls of workload `w` (after `warmup` untimed
    ones) with the dominant kernel stamped by HIP events, then profiles
    PROFILE_STEPS more calls stage by stage.  Returns (result dict, inputs)."""
    import torch

    import token_activation_perturbation_amd as dust
    from token_activation_perturbation_amd import roofline, synth

    dev = torch.device("cuda:0")
    inp = synth.make_inputs(w)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16

    def to_dev(name, cast=True):
        t = torch.from_numpy(inp[name]).to(dev)
        return (t.to(tdt) if cast else t).contiguous()

    if w.embedding:
        table, tg, ids = to_dev("table"), to_dev("target"), to_dev("ids", cast=False)
    elif w.attention:
        X, q, k, v = to_dev("X"), to_dev("q"), to_dev("k"), to_dev("v")
        E = to_dev("E", cast=False)
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
                dust.dust_attention_workspace_bytes(w.T, w.d_in, w.heads, w.d_head, w.seq_len,
                                                    w.site, w.K, w.antithetic)
                if w.attention else
                dust.dust_workspace_bytes_seq(w.T, w.d_in, w.d_out, w.seq_len, w.K, w.gamma,
                                              w.antithetic, dt_code))
    chain = not w.embedding and not w.head and not w.attention and ws_bytes > base_bytes
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    kw = dict(K=w.K, sigma=w.sigma, gamma=w.gamma, seed=w.noise_seed, antithetic=w.antithetic,
              seq_len=w.seq_len)
    if w.head:
        kw = dict(K=w.K, sigma=w.sigma, seed=w.noise_seed, antithetic=w.antithetic)

    def estimate(out):
        if w.embedding:
            return dust.dust_estimate_embedding(table, ids, tg, out=out, workspace=ws,
                                                scale=1.0 / w.T, **kw)
        if w.local:
            return dust.dust_estimate_local(X, E, out=out, workspace=ws, **kw)
        if w.attention:
            return dust.dust_estimate_attention(X, q, k, v, E, heads=w.heads, site=w.site,
                                                out=out, workspace=ws, **kw)
        if w.head:
            return dust.dust_estimate_head(X, W, labels, out=out, workspace=ws, **kw)
        return dust.dust_estimate(X, W, tg, out=out, workspace=ws, **kw)

    out = {}
    for _ in range(warmup):
        out = estimate(out)
    torch.cuda.synchronize(dev)
    if not bool(torch.isfinite(out["G_E" if w.embedding else "G_W"]).all()):
        sys.exit(f"bench.py: non-finite weight gradient on {w.name}")

    # event pairs stamped by the dispatch of the dominant kernel of every
    # timed step (the library launches it with hipExtLaunchKernelGGL)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for e in starts + stops:
        e.record()  # creates the underlying hipEvent
    torch.cuda.synchronize(dev)
    dust.dust_set_timing_events(starts, stops)

    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    wall0 = time.perf_counter()
    t_begin.record()
    for _ in range(steps):
        estimate(out)
    t_end.record()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    dust.dust_set_timing_events([], [])
    ms_per_step = t_begin.elapsed_time(t_end) / steps
    kernel_ms = sum(s.elapsed_time(e) for s, e in zip(starts, stops)) / steps

    # every stage, from a separate profiled pass (not the timed one)
    dust.dust_profile_begin(64 * PROFILE_STEPS)
    for _ in range(PROFILE_STEPS):
        estimate(out)
    records = dust.dust_profile_end()
    per = {}
    for r in records:
        e = per.setdefault(r["kernel"], {"ms": 0.0, "flops": 0.0, "bytes": 0.0, "calls": 0})
        e["ms"] += r["ms"]
        e["flops"] += r["flops"]
        e["bytes"] += r["bytes"]
        e["calls"] += 1
    stages = []
    for name, e in per.items():
        calls_per_step = e["calls"] / PROFILE_STEPS
        ms = e["ms"] / PROFILE_STEPS
        slots = None
        if name in roofline.NOISE_STAGES:
            slots = roofline.noise_stage_slots(name, w.T, w.d_out, w.K, w.antithetic,
                                               local=w.local) * calls_per_step
        elif name in ("attn_score_t_kernel", "attn_score_s_kernel"):
            bound, work, _, _ = roofline.attention_score_bound(
                w.site, w.T, w.seq_len, w.heads, w.d_head, w.K, w.antithetic)
            if bound == "alu":
                slots = work * calls_per_step

        st = roofline.stage_roofline(name, ms, e["flops"] / PROFILE_STEPS,
                                     e["bytes"] / PROFILE_STEPS, w.dtype, slots)
        st["calls"] = calls_per_step
        stages.append(st)
    stage_ms = sum(s["ms"] for s in stages)

    kernel = dominant_kernel(w, chain)
    bound, unit = "alu", "T lane-slot/s"
    if w.head:
        slots = roofline.head_kernel_slots(w.T, w.d_out, w.K, w.antithetic)
        min_s = roofline.head_min_seconds(w.T, w.d_out, w.K, w.antithetic)
        peak_per_s = roofline.PEAK_SLOTS_PER_S
    elif w.attention:
        # the score kernel's larger of its ALU and MFMA work; end to end,
        # that kernel at its bound plus the regeneration of every noise
        # value for g
        bound, slots, peak_per_s, unit = roofline.attention_score_bound(
            w.site, w.T, w.seq_len, w.heads, w.d_head, w.K, w.antithetic)
        min_s = (slots / peak_per_s + roofline.reweight_kernel_slots(
            w.T, w.d_out, w.K, w.antithetic) / roofline.PEAK_SLOTS_PER_S)
    else:
        slots = roofline.noise_stage_slots(kernel, w.T, w.d_out, w.K, w.antithetic,
                                           local=w.local)
        min_s = roofline.estimate_min_seconds(w.T, w.d_out, w.K, w.antithetic, local=w.local)
        peak_per_s = roofline.PEAK_SLOTS_PER_S
    achieved = slots / (kernel_ms * 1e-3) / 1e12
    peak = peak_per_s / 1e12
    res = {
        "workload": w.name,
        "value": w.rows / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step,
        "wall_ms_per_step": wall * 1e3 / steps,
        "roofline": {
            "bound": bound,
            "kernel": kernel,
            "kernel_ms": kernel_ms,
            "achieved": achieved,
            "peak": peak,
            "unit": unit,
            "frac": achieved / peak,
            "traffic": read_traffic(w.name, kernel),
            # one generation of every noise value at the ALU peak, over the step
            "end_to_end_frac": min_s / (ms_per_step * 1e-3),
            # every stage at the peak of its own bound, over the step
            "stages_bound_frac": sum(s["bound_ms"] for s in stages) / ms_per_step,
        },
        "stages": [{k: (round(v, 5) if isinstance(v, float) else v) for k, v in s.items()}
                   for s in stages],
        "profiled_ms_per_step": stage_ms,
    }
    return res, (inp if want_inputs else None)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE,
                    help="the headline workload (one of synth.py's)")
    ap.add_argument("--configs", default="all",
                    help="reference configurations measured besides the headline: 'all' (the "
                         "five), 'none', or a comma-separated list")
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
    if args.configs == "all":
        configs = list(REFERENCE_CONFIGS)
    elif args.configs == "none":
        configs = []
    else:
        configs = [c for c in args.configs.split(",") if c]
        bad = [c for c in configs if c not in synth.WORKLOADS]
        if bad:
            sys.exit(f"bench.py: unknown workload(s) {', '.join(bad)}; one of "
                     f"{', '.join(synth.WORKLOAD_ORDER)}")
    if args.steps < 1 or args.warmup < 0:
        sys.exit("bench.py: --steps must be >= 1 and --warmup >= 0")

    import torch

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    # an untimed plain copy of known size: rocprofv3's FETCH_SIZE / WRITE_SIZE
    # counters read on it calibrate the HBM bytes reported for our kernels
    cal_src = torch.ones(CAL_COPY_BYTES // 4, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize(dev)
    del cal_src, cal_dst

    head, inp = measure(w, args.steps, args.warmup, want_inputs=args.cpu_budget > 0)
    print(f"bench: {w.name} {head['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
    per_config = {}
    for name in configs:
        if name == w.name:
            r = head
        else:
            r, _ = measure(synth.WORKLOADS[name], args.steps, args.warmup)
            torch.cuda.empty_cache()
            print(f"bench: {name} {r['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
        cw = synth.WORKLOADS[name]
        per_config[name] = {
            "rows_per_s": r["value"], "ms_per_step": r["ms_per_step"],
            "config": cw.describe(),
            "dominant": {k: r["roofline"][k] for k in ("kernel", "kernel_ms", "frac",
                                                       "end_to_end_frac", "stages_bound_frac")},
            "stages": [{k: s[k] for k in ("kernel", "ms", "bound", "achieved", "unit", "frac",
                                          "hbm_frac")} for s in r["stages"]],
        }

    result = {
        "metric": ("slab-draw-token-rows/sec (K*T*V/256) for dust_estimate_head" if w.head else
                   "draw-token-rows/sec (K*T) for " +
                   ("dust_estimate_local" if w.local else
                    "dust_estimate_embedding" if w.embedding else
                    "dust_estimate_attention" if w.attention else "dust_estimate")),
        "value": head["value"],
        "unit": "draw-token-rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "wall_ms_per_step": head["wall_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "accumulation_dtype": "f32",
        "data": ("synthetic (seeded normal X and error estimate E; no dataset or trained weights)"
                 if w.local else
                 "synthetic (seeded normal X, cached q, k, v and error estimate E; no dataset or "
                 "trained weights)"
                 if w.attention else
                 "synthetic (seeded normal X, W and uniform labels; no dataset or trained weights)"
                 if w.head else
                 "synthetic (seeded normal table and target, Zipfian token ids; no dataset or "
                 "trained weights)"
                 if w.embedding else
                 "synthetic (seeded normal X, W, target; no dataset or trained weights)"),
        "config": {**w.describe(), "input_dtype": w.dtype, "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "stages": head["stages"],
        "configs": per_config,
    }
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
