#!/usr/bin/env python3
"""Benchmark of the MoL delta path on one MI355X.

One step = one layer pass of the whole path on one batch: align_block_size (remap inline)
+ the gate_up delta (shrink + expand, one fused launch) + the down delta. The default
workload is the decode layer of 23 tokens (hidden 2048, moe_intermediate 768, 128 experts,
top-8, 8 LoRA slots = 1024 virtual experts, rank 32, BLOCK_M 64).

Steps rotate over `--layers` independent layers (own weights, routing and activations,
seeded 0..L-1), as consecutive MoE layers of a model do, so a layer's weights are not
still in the 256 MiB MALL when it comes round again. Inputs are resident in HBM before
the timed region. Each layer's step is captured once into a hipGraph (torch.cuda.graph)
and the timed region replays them (`--mode eager` launches directly instead).

Prints one JSON line: routed pairs/s over the timed steps as `value`, microseconds per
layer, the roofline of the dominant kernel (the gate_up fused delta) from HIP events
around its launches inside the timed region, and the CPU oracle timed on the host cores
on a bounded sample of the same layers.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("µs/layer for align+shrink+expand at bs=23 decode; routed pairs/s; "
          "% HBM peak")
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--config", default="c1_decode_bs23")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle sample budget (0 = skip the CPU baseline)")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def layer_stats(dl):
    """Pairs, touched virtual experts and tokens of one layer, read from the GPU routing."""
    cfg = dl.cfg
    srt, eid, npp = dl.routing_host()
    blocks = srt.reshape(-1, cfg.block_m)
    real = blocks < cfg.numel
    valid_blocks = eid >= 0
    pairs = blocks[valid_blocks][real[valid_blocks]]
    P = int(pairs.size)
    D = int(np.unique(eid[valid_blocks]).size)
    T = int(np.unique(pairs // cfg.topk).size)
    return {"P": P, "D": D, "T": T, "npp": npp, "blocks": int(eid.size),
            "valid_blocks": int(valid_blocks.sum())}


def stage_bytes(cfg, st, stats):
    """Algorithmic HBM bytes of one stage's delta: every touched virtual expert's A and B
    once, the input rows the pairs read, and each pair's output row read and written,
    plus the routing entries of the real pairs and their blocks."""
    esz = 2 if cfg.dtype == "bf16" else 4
    P, D = stats["P"], stats["D"]
    rows = stats["T"] if st.input == "x" else P
    w = D * (st.R * st.K + st.N * st.r) * esz
    act = rows * st.K * esz
    out = 2 * P * st.N * esz
    idx = 4 * (P + stats["valid_blocks"])
    return w + act + out + idx


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for "
              f"--gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py runs on one GPU only (WORLD_SIZE > 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    from virtual_expert_routed_amd import configs, inputs
    from virtual_expert_routed_amd.layer import DeviceLayer

    cfg = configs.BY_NAME[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = max(1, args.layers)

    log(f"[bench] generating {L} layers of {cfg.name}")
    host_inputs, layers = [], []
    for l in range(L):
        inp = inputs.generate(cfg, seed=l)
        base = [inputs.base_out(cfg, si, seed=l) for si in range(len(cfg.stages))]
        layers.append(DeviceLayer(inp, device=dev, outs=base))
        host_inputs.append(inp)
    torch.cuda.synchronize()

    # warm-up (also fills the routing used for the byte model)
    log(f"[bench] warmup {args.warmup} steps")
    for i in range(max(1, args.warmup)):
        layers[i % L].run()
    torch.cuda.synchronize()
    stats = [layer_stats(dl) for dl in layers]

    def step_body(dl):
        dl.align()
        for si in range(len(cfg.stages)):
            dl.delta(si)

    graphs = None
    if args.mode == "graph":
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for dl in layers:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    step_body(dl)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for _ in range(2):
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()

    # ---- timed region: K steps, one layer each
    K = args.steps
    log(f"[bench] timing {K} steps ({args.mode})")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    if graphs is not None:
        for i in range(K):
            graphs[i % L].replay()
    else:
        for i in range(K):
            step_body(layers[i % L])
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_elapsed = ev0.elapsed_time(ev1) * 1e-3

    # ---- per-kernel times: HIP events around every launch, recorded on the launch stream.
    # A GPU sleep queued first lets the host enqueue all the steps ahead of the GPU, so
    # the events bracket back-to-back kernels rather than host launch latency.
    nt = max(L, min(K, 8 * L))
    nst = len(cfg.stages)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 2)] for _ in range(nt)]
    spacer_ms = 0.0
    if hasattr(torch.cuda, "_sleep"):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        torch.cuda._sleep(1 << 20)
        c1.record()
        torch.cuda.synchronize()
        per_cycle_ms = max(c0.elapsed_time(c1), 1e-3) / (1 << 20)
        spacer_ms = 30.0
        torch.cuda._sleep(int(spacer_ms / per_cycle_ms))
    for i in range(nt):
        dl = layers[i % L]
        e = evs[i]
        e[0].record()
        dl.align()
        e[1].record()
        for si in range(nst):
            dl.delta(si)
            e[2 + si].record()
    torch.cuda.synchronize()
    align_us = [evs[i][0].elapsed_time(evs[i][1]) * 1e3 for i in range(nt)]
    samples = [[evs[i][1 + si].elapsed_time(evs[i][2 + si]) * 1e3 for i in range(nt)]
               for si in range(nst)]
    stage_b = [[stage_bytes(cfg, st, stats[i % L]) for i in range(nt)] for st in cfg.stages]

    steps_P = sum(stats[i % L]["P"] for i in range(K))
    ms_per_step = elapsed / K * 1e3
    value = steps_P / elapsed
    dom = 0   # gate_up delta carries the most bytes
    dom_us = float(np.mean(samples[dom]))
    dom_bytes = float(np.mean(stage_b[dom]))
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    delta_us = sum(float(np.mean(samples[si])) for si in range(nst))
    delta_bytes = sum(float(np.mean(b)) for b in stage_b)
    timing_src = f"hip-events, eager launches queued behind a {spacer_ms:.0f} ms GPU sleep"

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "tokens": cfg.M, "hidden": cfg.hidden, "experts": cfg.E,
            "topk": cfg.topk, "lora_slots": cfg.S, "virtual_experts": cfg.V, "rank": cfg.rank,
            "block_m": cfg.block_m, "layers_rotated": L, "mode": args.mode,
            "accumulate": "fp32",
        },
        "us_per_layer": ms_per_step * 1e3,
        "us_per_layer_gpu_events": gpu_elapsed / K * 1e6,
        "align_us": float(np.mean(align_us)),
        "pairs_per_layer": float(np.mean([s["P"] for s in stats])),
        "touched_virtual_experts": float(np.mean([s["D"] for s in stats])),
        "delta_us": {st.name: float(np.mean(samples[si])) for si, st in enumerate(cfg.stages)},
        "delta_hbm_frac": delta_bytes / (delta_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "kernel_timing": timing_src,
        "roofline": {
            "kernel": f"delta_fused_kernel ({cfg.stages[dom].name})",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "bytes_per_launch": dom_bytes,
            "us_per_launch": dom_us,
        },
    }

    if args.cpu_seconds > 0:
        import oracle
        oracle.build()
        log(f"[bench] CPU oracle sample (~{args.cpu_seconds:.0f} s)")
        t0 = time.perf_counter()
        n_layers = n_pairs = 0
        while True:
            l = n_layers % L
            oracle.run_layer(host_inputs[l])
            n_layers += 1
            n_pairs += stats[l]["P"]
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": n_pairs / el, "unit": "pairs/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_layers} whole layer passes of {cfg.name} (layers 0..{L - 1} "
                      f"cycled), fp64 C oracle, {el:.1f} s",
            "us_per_layer": el / n_layers * 1e6,
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
