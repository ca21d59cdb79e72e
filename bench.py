"""Benchmark of one EP rank's fixed-pool, three-wave MoE layer on one MI355X.

One step = the whole layer for one batch: route -> pack into 64 fixed send
pools -> (self-block of the dispatch exchange) -> 3 waves of receive + expert
SwiGLU GEMMs -> (self-block of the return exchange) -> combine + up-projection
+ shared experts.  Inputs are resident in HBM before timing starts.  The
metric is routed token-assignments per second: T * k / step time.

Prints ONE JSON line.  Options: --steps K --warmup W --config {2,3,4,5}
--gather {fused,buffer} --no-cpu-baseline --cpu-tokens N.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "routed token-assignments/s per GPU (dispatch+expert+combine); HBM GB/s, MFMA %"
PEAK_MFMA_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--gather", choices=["fused", "buffer"], default="fused")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    return ap.parse_args()


def cpu_baseline(cfg, seed, tokens):
    """Time the CPU oracle on the same workload with fewer tokens per rank."""
    from oracle import moe_oracle as O
    from workload import configs, gen
    sh = configs.with_tokens(configs.get(cfg), tokens)
    scap, _ = O.capacities(sh)
    inp = gen.generate(sh, seed=seed, send_cap=scap)
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("internal_api") in ("openblas", "mkl", "blis")]
        if info:
            threads = int(info[0]["num_threads"])
    except Exception:
        pass
    t0 = time.perf_counter()
    O.layer_one_rank(sh, inp, with_floats=True)
    dt = time.perf_counter() - t0
    return {"value": tokens * sh.top_k / dt, "unit": "assignments/s", "cores": threads, "kind": "oracle",
            "sample": f"{sh.name}: the same layer with {tokens} tokens per rank (send pools {scap} rows), "
                      f"full float64 oracle, {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU: one EP rank's share of the layer at its real "
                                   "shape; runs on more than one GPU are not part of it", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from workload import configs, gen
    from grouped_expert_ffn_router_amd import binding, runner

    sh = configs.get(args.config)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    scap, rcap, _ = binding.capacity(binding.make_dims(sh))
    inp = gen.generate(sh, seed=args.seed, send_cap=scap)
    lay = runner.OneRankLayer(sh, inp, device=dev, gather=args.gather)
    del inp
    stream = torch.cuda.current_stream()
    full = sh.layer == "full"

    def step(ev=None):
        # events between the C-ABI calls time each call on the stream it runs on
        def mark(name):
            if ev is not None:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                ev.append((name, e))
        mark("start")
        lay.dispatch(stream)
        mark("dispatch")
        for w in range(sh.waves):
            lay.receive_wave(w, stream)
            mark(f"recv{w}")
            if full:
                lay.expert_wave(w, stream)
                mark(f"expert{w}")
        if full:
            lay.combine(stream)
            mark("combine")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # whole-step timing
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    # per-call timing (separate pass, events between calls)
    per = {}
    for _ in range(args.steps):
        ev = []
        step(ev)
        torch.cuda.synchronize()
        for (a, ea), (b, eb) in zip(ev[:-1], ev[1:]):
            key = b if not b[-1].isdigit() else b[:-1]
            per.setdefault(key, []).append(ea.elapsed_time(eb))
    rep = lay.drop_report(stream)
    T, k, L, H = sh.tokens, sh.top_k, sh.latent, sh.expert_hidden
    value = T * k / (ms * 1e-3)
    waves_rows = lay.wave_count.sum(dim=1).cpu().numpy()
    # per-call average per launch
    brk = {key: float(np.mean(v)) for key, v in per.items()}
    out = {
        "metric": METRIC, "value": value, "unit": "assignments/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": sh.act, "data": "synthetic",
        "config": {"workload": sh.name, "tokens_per_rank": T, "d_model": sh.d_model, "latent": L,
                   "experts": sh.n_experts, "top_k": k, "ep_ranks": sh.n_ranks, "local_experts": sh.local_experts,
                   "waves": sh.waves, "expert_hidden": H, "shared_experts": sh.shared_experts,
                   "shared_hidden": sh.shared_hidden, "send_cap": scap, "recv_cap": rcap,
                   "gather": args.gather, "parallelism": "ep64, one rank's share"},
        "breakdown_ms": brk,
        "drops": {"send_dropped": rep["send_dropped"], "recv_dropped": rep["recv_dropped"],
                  "recv_kept": rep["recv_kept"], "send_kept": rep["send_kept"]},
    }
    if full:
        # dominant step: the grouped SwiGLU expert GEMMs (moe_expert_gemm), per wave launch
        rows = float(np.mean(waves_rows))
        flops = 6.0 * L * H * rows
        t_ms = brk["expert"]
        ach = flops / (t_ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": ach, "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / PEAK_MFMA_BF16_TFLOPS, "traffic": None,
                           "kernel": "moe_expert_gemm (gate/up + down GEMMs of one wave, 2 experts)",
                           "work_per_launch": f"6*L*H flops x {rows:.0f} kept rows"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config, args.seed, args.cpu_tokens)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
