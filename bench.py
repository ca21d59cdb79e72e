"""Benchmark of one EP rank's fixed-pool, three-wave MoE layer on one MI355X.

One step = the whole layer for one batch of the rank's tokens: route (router
+ latent down-projection GEMM, top-k select) -> pack into the 64 fixed send
pools -> (self-block of the dispatch exchange) -> receive ranking -> 3 waves of
placement + expert SwiGLU GEMMs (rows scattered into the return pools; odd
waves on a second stream) -> (self-block of the return exchange) -> weighted
combine + up-projection + shared experts (their gate/up GEMM on the second
stream).  The
pools the other 63 ranks send, and the rows they return, are seeded inputs
resident in HBM before timing starts.  The metric is routed
token-assignments per second: T * k / step time.

Prints ONE JSON line with, besides the contract fields:
  roofline      the dominant kernel (largest summed time) against its peak,
                timed live with HIP events on the stream it runs on
                (moe_timing_*), with HBM traffic from the committed rocprofv3
                counter summary when that summary matches the current sources
  kernels       every kernel's average duration and roofline fraction
  cpu_baseline  the CPU oracle timed on a bounded sample of the same layer

Options: --steps K --warmup W --config {2,3,4,5,6} --gather {fused,buffer} --streams {1,2}
--sweep-capacity (one line per capacity-factor point instead of the benchmark line),
--dropless (capacities fitted to the exchanged counts against the fixed factors),
--vendor-gemm (torch's bf16 matmul on the layer's GEMM shapes, a reference point for the GEMM core)
--graph (the step captured once as a HIP graph, its replays timed)
--no-cpu-baseline --cpu-tokens N --seed S.  --gpus N > 1 exits: the benchmark
measures one GPU.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed token-assignments/s per GPU (dispatch+expert+combine); HBM GB/s, MFMA %"
PEAK_MFMA_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
SOURCES = ["grouped_expert_ffn_router_amd/csrc/api.hip", "grouped_expert_ffn_router_amd/csrc/kernels.hip",
           "grouped_expert_ffn_router_amd/csrc/gemm.h", "grouped_expert_ffn_router_amd/csrc/moe_common.h",
           "grouped_expert_ffn_router_amd/csrc/moe_internal.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--gather", choices=["fused", "buffer"], default="fused")
    ap.add_argument("--streams", type=int, choices=[1, 2], default=2,
                    help="2: the shared experts and the odd waves run on a second stream, beside the routed "
                         "path and the even waves")
    ap.add_argument("--live-waves", type=int, default=2,
                    help="waves whose scratch (SwiGLU hidden rows, partial tiles) the workspace holds at once; "
                         "2 (default): two waves overlap, one on each stream, as many as two streams can run; "
                         "1: one wave live at a time, waves in order; 0: all waves")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (both streams) as a HIP graph after the warm-up and time its replays")
    ap.add_argument("--cpu-runs", type=int, default=0,
                    help="timed runs of the CPU oracle (the median is reported); 0: 3, or 1 for 65,536 tokens")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens per rank of the CPU-oracle sample (0: the whole workload)")
    ap.add_argument("--sweep-capacity", action="store_true",
                    help="instead of the benchmark line: one JSON line per (send, receive) capacity factor "
                         "with drop rates, exchange memory and throughput")
    ap.add_argument("--dropless", action="store_true",
                    help="instead of the benchmark line: the layer with capacities fitted exactly to the "
                         "exchanged counts (no drops) against the fixed factors, one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="instead of the benchmark line: torch's bf16 matmul (the vendor GEMM library) on the "
                         "layer's GEMM shapes with N(0,1) operands, one JSON line per shape (a reference point "
                         "for the GEMM core, to be profiled with the same counters)")
    return ap.parse_args()


def source_digest():
    h = hashlib.sha256()
    for p in SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel, workload):
    """HBM bytes per launch from profiles/<kernel>_<workload>_pmc.txt, if that
    summary was taken from the current sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_work(sh, kept_rows_per_wave, send_kept, send_cap):
    """Algorithmic flops (GEMMs) or bytes (data movement) of one launch of each kernel.

    GEMMs count 2*M*N*K over the rows the layer keeps (never capacity padding);
    data-movement kernels count the bytes the method must move."""
    T, D, L, E, k, R = sh.tokens, sh.d_model, sh.latent, sh.n_experts, sh.top_k, sh.n_ranks
    H, S, HS = sh.expert_hidden, sh.shared_experts, sh.shared_hidden
    es = 2 if sh.act == "bf16" else 4
    rows = float(np.mean(kept_rows_per_wave)) if len(kept_rows_per_wave) else 0.0
    return {
        "route_gemm": ("flop", 2.0 * T * (E + L) * D),
        "expert_gate_up": ("flop", 2.0 * rows * 2 * H * L),
        "expert_down": ("flop", 2.0 * rows * L * H),
        "shared_gate_up": ("flop", 2.0 * T * 2 * S * HS * D),
        "up_shared_down": ("flop", 2.0 * T * D * (L + S * HS)),
        # read z once, write each kept row (payload + id), ids of empty slots,
        # read top-k ids, write slot_of
        "pack": ("byte", T * L * es + send_kept * (L * es + 4) + 4.0 * (R * send_cap - send_kept) + 8.0 * T * k),
        # read every returned row of the rank's kept assignments, the weights
        # and slots, write c
        "combine": ("byte", send_kept * L * es + 8.0 * T * k + T * L * es),
    }


def cpu_baseline(cfg, seed, tokens, runs):
    """Time the CPU oracle on a bounded sample: the same layer at `tokens` tokens per rank
    (median of `runs` runs)."""
    from oracle import moe_oracle as O
    from workload import configs, gen
    base = configs.get(cfg)
    sh = configs.with_tokens(base, tokens) if tokens != base.tokens else base
    scap, _ = O.capacities(sh)
    inp = gen.generate(sh, seed=seed, send_cap=scap)
    if "sources" in inp:  # the other ranks' pools: their dispatch is not this rank's work (untimed)
        inp["foreign_ids"], inp["foreign_rows"], _ = O.routed_source_pools(sh, inp, with_rows=sh.layer == "full")
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("internal_api") in ("openblas", "mkl", "blis")]
        if info:
            threads = int(info[0]["num_threads"])
    except Exception:
        pass
    times = []
    for _ in range(max(runs, 1)):
        t0 = time.perf_counter()
        O.layer_one_rank(sh, inp, with_floats=True)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    what = "route + pack + receive" if sh.layer != "full" else "the full layer"
    scope = (f"the whole {base.name} workload" if tokens == base.tokens else
             f"the {base.name} recipe at {tokens} tokens per rank (send pools of {scap} rows)")
    return {"value": tokens * sh.top_k / dt, "unit": "assignments/s", "cores": threads, "kind": "oracle",
            "sample": f"{scope}: {what} of one rank in the float64 oracle (seed {seed}), input generation "
                      f"excluded, median of {len(times)} run(s): " + ", ".join(f"{t:.2f}" for t in times) + " s",
            "runs_s": times,
            "host": {"cpu_model": _cpu_model(), "logical_cpus": os.cpu_count()}}


def reference_rates(dev):
    """What the device reaches outside this library, measured in the same run:
    a plain device-to-device copy of 1 GiB (read + write bytes / time) and the
    vendor bf16 GEMM (torch.matmul, hipBLASLt) on 8192^3 with N(0,1) operands."""
    import torch
    a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        b.copy_(a)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy = 2 * a.numel() * 2 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    n = 8192
    x = torch.randn(n, n, device=dev).to(torch.bfloat16)
    y = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(3):
        c = x @ y
    e0.record()
    for _ in range(10):
        c = x @ y
    e1.record()
    torch.cuda.synchronize()
    gemm = 2 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, y, c
    torch.cuda.empty_cache()
    return {"device_copy_GBs": copy, "vendor_bf16_gemm_8192_TFLOPs": gemm}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


SWEEP_FACTORS = [(110, 115), (100, 115), (125, 115), (150, 115), (110, 100), (110, 130), (110, 150)]


VENDOR_SHAPES = [(22528, 3072, 3072), (8192, 6144, 6144), (8192, 6144, 3072), (8192, 3456, 6144),
                 (22528, 3072, 1536)]


def vendor_gemm(args):
    """torch.matmul in bf16 (the vendor library) on M x N x K shapes of the layer:
    one expert wave's gate/up rows as one dense GEMM, the shared gate/up, the
    up-projection + shared down, the route GEMM, one expert wave's down rows.  B is a transposed view of an
    [N][K] matrix (2-D matmul, no batching)."""
    import torch
    torch.manual_seed(args.seed)
    for M, N, K in VENDOR_SHAPES:
        a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        b = torch.randn(N, K, device="cuda").to(torch.bfloat16)
        bt = b.t()
        for _ in range(args.warmup):
            c = a @ bt
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            c = a @ bt
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        print(json.dumps({"vendor_gemm": "torch.matmul bf16", "M": M, "N": N, "K": K, "ms": ms,
                          "tflops": 2 * M * N * K / (ms * 1e-3) / 1e12}), flush=True)
        del a, b, bt, c


def capacity_sweep(args):
    """Capacity factors vs drops, exchange memory and throughput (factors in percent).

    The other ranks' tokens are drawn once and reused at every point; each
    point rebuilds the layer (pools, returns and workspace sized by its
    capacities) and times args.steps steps after args.warmup."""
    from dataclasses import replace
    import torch
    from workload import configs, gen
    from grouped_expert_ffn_router_amd import binding, runner
    base = configs.get(args.config)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    drawn = None
    for sn, rn in SWEEP_FACTORS:
        sh = replace(base, send_num=sn, send_den=100, recv_num=rn, recv_den=100)
        dims = binding.make_dims(sh)
        scap, rcap, prow = binding.capacity(dims)
        inp = gen.generate(sh, seed=args.seed, send_cap=scap)
        if "sources" in inp:
            if drawn is None:
                drawn = {s: inp["sources"](s) for s in range(sh.n_ranks)}
            inp["sources"] = drawn.__getitem__
        lay = runner.OneRankLayer(sh, inp, device="cuda:0", gather=args.gather, live_waves=args.live_waves)
        del inp
        full = sh.layer == "full"
        side = torch.cuda.Stream() if args.streams == 2 and full else None
        for _ in range(args.warmup):
            lay.run(stream, side)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            lay.run(stream, side)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        rep = lay.drop_report(stream)
        es = 2 if sh.act == "bf16" else 4
        pools = 2 * sh.n_ranks * scap * prow                          # send + receive pools
        rets = 2 * sh.n_ranks * scap * sh.latent * es if full else 0   # returned rows, both ways
        n_assign = sh.tokens * sh.top_k
        print(json.dumps({
            "sweep": "capacity", "workload": base.name, "send_factor": sn / 100, "recv_factor": rn / 100,
            "send_cap": scap, "recv_cap": rcap,
            "send_drop_rate": rep["send_dropped"] / n_assign,
            "recv_drop_rate": rep["recv_dropped"] / max(sum(rep["expert_arrivals"]), 1),
            "send_dropped": rep["send_dropped"], "recv_dropped": rep["recv_dropped"],
            "exchange_bytes": pools + rets, "workspace_bytes": binding.workspace_size(dims),
            "ms_per_step": ms, "assignments_per_s": n_assign / (ms * 1e-3)}), flush=True)
        del lay
        torch.cuda.empty_cache()


def dropless(args):
    """Fixed capacity factors against capacities fitted exactly to the counts.

    A dropless exchange first sends each destination its row count; with the
    counts known, every pool can be sized to the largest demand and every
    expert's bank to its largest arrivals, so nothing is dropped.  Three builds
    of the one-rank layer (the other ranks' tokens drawn once): the fixed
    factors (timed; its counts give the pool size), the exact send cap with a
    receive cap no arrival can exceed (its arrivals give the bank size), and
    both caps exact (timed, drop-free); then the ragged layout, whose pools
    are laid end to end and hold exactly the rows sent (timed, drop-free)."""
    import torch
    from workload import configs, gen
    from grouped_expert_ffn_router_amd import binding, runner
    base = configs.get(args.config)
    if base.foreign != "routed":
        raise SystemExit("--dropless needs a workload whose other ranks route their own tokens (configs 2, 3, 4, 6)")
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    drawn = {}

    def inputs(sh):
        scap, _, _ = binding.capacity(binding.make_dims(sh))
        inp = gen.generate(sh, seed=args.seed, send_cap=scap)
        if not drawn:
            drawn.update({s: inp["sources"](s) for s in range(sh.n_ranks)})
        inp["sources"] = drawn.__getitem__
        return inp

    def build(sh):
        return runner.OneRankLayer(sh, inputs(sh), device="cuda:0", gather=args.gather, live_waves=args.live_waves)

    def measure(lay, timed):
        side = torch.cuda.Stream() if args.streams == 2 and lay.full else None
        for _ in range(args.warmup if timed else 1):
            lay.run(stream, side)
        torch.cuda.synchronize()
        ms = None
        if timed:
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(args.steps):
                lay.run(stream, side)
            t1.record(stream)
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / args.steps
        return ms, lay.drop_report(stream)

    def footprint(sh, lay):
        es = 2 if sh.act == "bf16" else 4
        rets = 2 * sh.n_ranks * lay.scap * sh.latent * es if lay.full else 0
        return 2 * sh.n_ranks * lay.scap * lay.prow + rets + binding.workspace_size(lay.dims)

    n_assign = base.tokens * base.top_k
    lay = build(base)
    ms_fixed, rep = measure(lay, True)
    fixed = {"send_cap": lay.scap, "recv_cap": lay.rcap, "send_dropped": rep["send_dropped"],
             "recv_dropped": rep["recv_dropped"], "bytes": footprint(base, lay), "ms_per_step": ms_fixed}
    pool_rows = max(max(rep["send_demand"]), max(lay.source_demand.values(), default=0))
    del lay
    torch.cuda.empty_cache()
    lay = build(configs.exact_fit(base, pool_rows, base.n_ranks * pool_rows))
    _, rep = measure(lay, False)
    expert_rows = max(rep["expert_arrivals"])
    del lay
    torch.cuda.empty_cache()
    sh = configs.exact_fit(base, pool_rows, expert_rows)
    lay = build(sh)
    ms_fit, rep = measure(lay, True)
    fit = {"send_cap": lay.scap, "recv_cap": lay.rcap, "send_dropped": rep["send_dropped"],
           "recv_dropped": rep["recv_dropped"], "bytes": footprint(sh, lay), "ms_per_step": ms_fit}
    del lay
    torch.cuda.empty_cache()
    # ragged pools: laid end to end by destination, as long as the counts
    lay = runner.RaggedOneRankLayer(base, inputs(sh), expert_rows, device="cuda:0", gather=args.gather,
                                    live_waves=args.live_waves)
    ms_rag, rep = measure(lay, True)
    rag = {"rows_sent": int(lay.own_off[-1]), "rows_received": lay.n_recv, "recv_cap": lay.rcap,
           "wave_rows": lay.wave_rows, "send_dropped": rep["send_dropped"], "recv_dropped": rep["recv_dropped"],
           "bytes": lay.footprint(), "workspace_bytes": lay.ws.numel(), "ms_per_step": ms_rag}
    del lay
    torch.cuda.empty_cache()
    # the same ragged exchange with a bank of expert_rows hidden rows per expert
    lay = runner.RaggedOneRankLayer(base, inputs(sh), expert_rows, device="cuda:0", gather=args.gather,
                                    ragged_banks=False, live_waves=args.live_waves)
    ms_rag_fixed, _ = measure(lay, True)
    rag["fixed_banks"] = {"bytes": lay.footprint(), "workspace_bytes": lay.ws.numel(), "ms_per_step": ms_rag_fixed}
    print(json.dumps({"comparison": "dropless (capacities fitted to the exchanged counts; ragged pools) vs fixed "
                                    "factors", "workload": base.name, "fixed": fixed, "dropless": fit,
                      "ragged": rag,
                      "fixed_assignments_per_s": n_assign / (ms_fixed * 1e-3),
                      "dropless_assignments_per_s": n_assign / (ms_fit * 1e-3),
                      "ragged_assignments_per_s": n_assign / (ms_rag * 1e-3)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU: one EP rank's share of the layer at its real "
                                   "shape; multi-GPU runs are not part of it", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.sweep_capacity:
        capacity_sweep(args)
        return
    if args.dropless:
        dropless(args)
        return
    if args.vendor_gemm:
        vendor_gemm(args)
        return
    import torch
    from workload import configs, gen
    from grouped_expert_ffn_router_amd import binding, runner

    sh = configs.get(args.config)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    scap, rcap, _ = binding.capacity(binding.make_dims(sh))
    inp = gen.generate(sh, seed=args.seed, send_cap=scap)
    lay = runner.OneRankLayer(sh, inp, device=dev, gather=args.gather, live_waves=args.live_waves)
    del inp
    stream = torch.cuda.current_stream()
    full = sh.layer == "full"
    side = torch.cuda.Stream() if args.streams == 2 and full else None

    for _ in range(args.warmup):
        lay.run(stream, side)
    torch.cuda.synchronize()
    step = lambda: lay.run(stream, side)
    if args.graph:
        # one step captured as a HIP graph (the side stream forks from and
        # joins the capture stream inside it; the step allocates nothing and
        # records no memset) and replayed on a stream of its own
        graph, main = torch.cuda.CUDAGraph(), torch.cuda.Stream()
        main.wait_stream(stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=main):
            lay.run(main, side)
        torch.cuda.synchronize()
        stream = main

        def step():
            with torch.cuda.stream(main):
                graph.replay()

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
    # an event on the main stream before every step and after the last: a
    # step's combine waits for its side-stream work, and the next step's
    # side-stream work waits for that combine, so consecutive events bracket
    # exactly one step
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]

    # per-kernel pass, all on one stream so that no two kernels share the
    # chip: every library launch bracketed by HIP events on its stream
    binding.timing_read()
    binding.timing_enable(True)
    for _ in range(args.steps):
        lay.run(stream)
    torch.cuda.synchronize()
    per = binding.timing_read()
    binding.timing_enable(False)

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    rates = reference_rates(dev)

    rep = lay.drop_report(stream)
    T, k = sh.tokens, sh.top_k
    kept_waves = lay.wave_count.sum(dim=1).cpu().numpy() if full else np.zeros(0)
    work = algorithmic_work(sh, kept_waves, rep["send_kept"], scap)
    kernels = {}
    for name, (n, tot) in per.items():
        avg = tot / max(n, 1)
        ent = {"launches_per_step": n / args.steps, "avg_ms": avg}
        if name in work and avg > 0:
            kind, amount = work[name]
            if kind == "flop":
                ach = amount / (avg * 1e-3) / 1e12
                ent.update(unit="TFLOP/s", achieved=ach, frac=ach / PEAK_MFMA_BF16_TFLOPS)
            else:
                ach = amount / (avg * 1e-3) / 1e9
                ent.update(unit="GB/s", achieved=ach, frac=ach / PEAK_HBM_GBS)
        kernels[name] = ent
    dom = max(per, key=lambda n: per[n][1])
    d = kernels[dom]
    kind = work[dom][0] if dom in work else None
    out = {
        "metric": METRIC, "value": T * k / (ms * 1e-3), "unit": "assignments/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "step_ms": {"mean": ms, "median": float(np.median(step_ms)), "min": float(np.min(step_ms)),
                    "max": float(np.max(step_ms))},
        "kept_assignments_per_s": rep["send_kept"] / (ms * 1e-3),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if sh.act == "bf16" else "f32",
        "data": "synthetic (seeded; shapes of the pages' 4K-context expert layer)",
        "config": {"workload": sh.name, "tokens_per_rank": T, "d_model": sh.d_model, "latent": sh.latent,
                   "experts": sh.n_experts, "top_k": k, "ep_ranks": sh.n_ranks, "local_experts": sh.local_experts,
                   "waves": sh.waves, "expert_hidden": sh.expert_hidden, "shared_experts": sh.shared_experts,
                   "shared_hidden": sh.shared_hidden, "send_cap": scap, "recv_cap": rcap, "gather": args.gather,
                   "live_waves": lay.live_waves, "streams": args.streams if full else 1, "hip_graph": args.graph,
                   "parallelism": "one EP rank of 64 (the other ranks' pools and returns are inputs)"},
    }
    if kind is not None:
        traffic = committed_traffic(dom, sh.name)
        ceiling = rates["vendor_bf16_gemm_8192_TFLOPs"] if kind == "flop" else rates["device_copy_GBs"]
        out["roofline"] = {"bound": "mfma" if kind == "flop" else "hbm", "achieved": d["achieved"],
                           "peak": PEAK_MFMA_BF16_TFLOPS if kind == "flop" else PEAK_HBM_GBS, "unit": d["unit"],
                           "frac": d["frac"], "traffic": traffic, "kernel": dom, "avg_ms": d["avg_ms"],
                           "work_per_launch": work[dom][1], "work_unit": kind,
                           "measured_ceiling": ceiling, "frac_of_measured_ceiling": d["achieved"] / ceiling}
    for name, ent in kernels.items():
        if ent.get("unit") == "GB/s":
            ent["frac_of_device_copy"] = ent["achieved"] / rates["device_copy_GBs"]
        elif ent.get("unit") == "TFLOP/s":
            ent["frac_of_vendor_gemm"] = ent["achieved"] / rates["vendor_bf16_gemm_8192_TFLOPs"]
    out["kernels"] = kernels
    out["reference_rates"] = rates
    out["memory"] = lay.memory()
    out["drops"] = {"send_dropped": rep["send_dropped"], "recv_dropped": rep["recv_dropped"],
                    "send_kept": rep["send_kept"], "recv_kept": rep["recv_kept"]}
    out["source_digest"] = source_digest()
    if not args.no_cpu_baseline:
        ctok = min(args.cpu_tokens, sh.tokens) if args.cpu_tokens else sh.tokens
        runs = args.cpu_runs if args.cpu_runs else (1 if ctok >= 65536 else 3)
        out["cpu_baseline"] = cpu_baseline(args.config, args.seed, ctok, runs)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
