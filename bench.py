#!/usr/bin/env python3
"""Benchmark of the MoL delta path on one MI355X.

One step = one layer pass of the whole path on one batch: align_block_size (remap inline)
+ the gate_up delta (shrink + expand) + the down delta (shrink + expand). The default
workload is the decode layer of 23 tokens (hidden 2048, moe_intermediate 768, 128 experts,
top-8, 8 LoRA slots = 1024 virtual experts, rank 32, BLOCK_M 64).

Steps rotate over `--layers` independent layers (own weights, routing and activations,
seeded 0..L-1), as consecutive MoE layers of a model do, so a layer's weights are not
still in the 256 MiB MALL when it comes round again. Inputs are resident in HBM before
the timed region. Each layer's step is captured once into a hipGraph (torch.cuda.graph)
and the timed region replays them (`--mode eager` launches directly instead).

Prints one JSON line: routed pairs/s over the timed steps as `value`, microseconds per
layer, per-kernel times and the roofline of the dominant (longest) kernel from HIP events
around its launches, and the CPU oracle timed on the host cores on a bounded sample of
the same layers.
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
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="accepted for older profile commands: the 2 GiB copy that measures "
                         "the achievable peak (and calibrates the counters) always runs")
    ap.add_argument("--no-floor", action="store_true",
                    help="skip the read-only streaming probe at the delta kernels' shapes")
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
    # runs of up to four consecutive blocks of one virtual expert (the align's work plan)
    v = eid[valid_blocks]
    runs = int(sum(-(-int(c) // 4) for c in np.unique(v, return_counts=True)[1])) if v.size \
        else 0
    return {"P": P, "D": D, "T": T, "npp": npp, "blocks": int(eid.size),
            "valid_blocks": int(valid_blocks.sum()), "runs": runs}


def _sizes(cfg, st, stats):
    esz = 2 if cfg.dtype == "bf16" else 4
    rows = stats["T"] if st.input == "x" else stats["P"]
    idx = 4 * (stats["P"] + stats["valid_blocks"])
    return esz, rows, idx


def stage_bytes(cfg, st, stats):
    """Algorithmic HBM bytes of one stage's delta: every touched virtual expert's A and B
    once, the input rows the pairs read, and each pair's output row read and written,
    plus the routing entries of the real pairs and their blocks. The fp32 rank-space
    intermediate s is not counted: a fused delta need not move it through HBM."""
    esz, rows, idx = _sizes(cfg, st, stats)
    P, D = stats["P"], stats["D"]
    return D * (st.R * st.K + st.N * st.r) * esz + rows * st.K * esz \
        + 2 * P * st.N * esz + idx


def shrink_bytes(cfg, st, stats):
    """Algorithmic bytes of one shrink launch: A of every touched virtual expert, the
    input rows, the fp32 s rows it writes, and the routing entries."""
    esz, rows, idx = _sizes(cfg, st, stats)
    return stats["D"] * st.R * st.K * esz + rows * st.K * esz + stats["P"] * st.R * 4 + idx


def expand_bytes(cfg, st, stats):
    """Algorithmic bytes of one expand launch: B of every touched virtual expert, the
    fp32 s rows, each pair's output row read and written, and the routing entries."""
    esz, _, idx = _sizes(cfg, st, stats)
    P = stats["P"]
    return stats["D"] * st.N * st.r * esz + P * st.R * 4 + 2 * P * st.N * esz + idx


def combine_bytes(cfg, st, n_local):
    """Algorithmic bytes of one combine launch: the rows of the pairs with a local expert
    read once, the per-token output written, and the ids and weights."""
    esz = 2 if cfg.dtype == "bf16" else 4
    return n_local * st.N * esz + cfg.M * st.N * esz + cfg.numel * 8


def fused_combine_bytes(cfg, st, stats, n_local):
    """Algorithmic bytes of one fused down expand + combine: B of every touched virtual
    expert, the fp32 s rows, the base rows of the local pairs, the per-token output, and
    the ids, slots and weights. The per-pair rows are neither read back nor written."""
    esz = 2 if cfg.dtype == "bf16" else 4
    return (stats["D"] * st.N * st.r * esz + stats["P"] * st.R * 4 + n_local * st.N * esz
            + cfg.M * st.N * esz + cfg.numel * 8 + cfg.M * 4)


def shrink_rows_per_item(cfg, st):
    """Rows of A_v per VALU shrink item: from 4, doubled while two such items' rows fit
    32 KiB, at most 32."""
    esz = 2 if cfg.dtype == "bf16" else 4
    rpi = 4
    while rpi < 32 and rpi * 2 * st.K * esz <= 32768:
        rpi *= 2
    return rpi


def grid_report(cfg, max_blocks, stats):
    """Workgroups each kernel launches (the grid follows the block bound, not padded rows)
    and how many of them belong to live blocks with a virtual expert, per stage. Where the
    MFMA kernels take the batch, theirs are listed instead (items: blocks times row tiles
    for the shrink, the plan's run room times column chunks for the expand; the grids are
    rounded up to a multiple of 8)."""
    vb = float(np.mean([s["valid_blocks"] for s in stats]))
    rep = {}
    for st in cfg.stages:
        rg = -(-st.R // shrink_rows_per_item(cfg, st))
        nch = -(-st.N // 256)
        if "mfma" in kernel_name(cfg, st, "shrink"):
            rt = -(-st.R // (128 if st.R > 64 else 64))
            rep[f"shrink {st.name}"] = {"launched": -(-max_blocks * rt // 8) * 8,
                                        "live_blocks_items": vb * rt}
        else:
            rep[f"shrink {st.name}"] = {"launched": max_blocks * rg,
                                        "live_blocks_items": vb * rg}
        if "mfma" in kernel_name(cfg, st, "expand"):
            runs = min(max_blocks, cfg.numel)
            rep[f"expand {st.name}"] = {"launched": -(-runs * nch // 8) * 8,
                                        "live_runs_items": float(np.mean(
                                            [s["runs"] for s in stats])) * nch}
        else:
            rep[f"expand {st.name}"] = {"launched": max_blocks * nch,
                                        "live_blocks_items": vb * nch}
    return rep


def base_gemm_leg(cfg, layers, host_inputs, torch, n_layers=2, rounds=8):
    """The base grouped GEMM of each stage, alone and with the LoRA delta fused into its
    epilogue, beside the unfused pair (base GEMM, then the LoRA expand into the same rows).
    Two layers rotate (their touched base weights, ~0.9 GB each at the decode configs, are far
    beyond the MALL); HIP events around runs of one call per layer, as for the path's
    kernels. Reported beside the headline, not part of it."""
    from virtual_expert_routed_amd import inputs
    use = layers[:min(n_layers, len(layers))]
    for l, dl in enumerate(use):
        dl.attach_base([inputs.base_weights(cfg, si, l) for si in range(len(cfg.stages))])
        dl.align()
        dl.align_base()
        for si in range(len(cfg.stages)):
            dl.shrink(si)
    torch.cuda.synchronize()
    esz = 2 if cfg.dtype == "bf16" else 4
    res = {}
    for si, st in enumerate(cfg.stages):
        fns = {"base": lambda dl: dl.base_gemm(si, False),
               "expand": lambda dl: dl.expand(si),
               "fused": lambda dl: dl.base_gemm(si, True)}
        for fn in fns.values():  # warm
            for dl in use:
                fn(dl)
        ev = {k: [] for k in fns}
        for _ in range(rounds):
            for k, fn in fns.items():
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for dl in use:
                    fn(dl)
                b.record()
                ev[k].append((a, b))
        torch.cuda.synchronize()
        us = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) * 1e3 / len(use)
              for k, v in ev.items()}
        # algorithmic bytes: touched base experts' W, input rows, each local pair's out row
        # written (the fused form adds the LoRA B of the touched virtual experts and s)
        byt, fbyt = [], []
        for h in host_inputs[:len(use)]:
            t = h.topk_ids.reshape(-1)
            loc = (t >= 0) & (t < cfg.E)
            nexp = int(np.unique(t[loc]).size)
            rows = int(np.unique(np.nonzero(loc)[0] // cfg.topk).size) if st.input == "x" \
                else int(loc.sum())
            b0 = nexp * st.N * st.K * esz + rows * st.K * esz + int(loc.sum()) * st.N * esz
            v = t + np.repeat(h.lora_ids, cfg.topk) * cfg.E
            lv = loc & (np.repeat(h.lora_ids, cfg.topk) >= 0) & (np.repeat(h.lora_ids, cfg.topk) < cfg.S)
            d = int(np.unique(v[lv]).size)
            byt.append(b0)
            fbyt.append(b0 + d * st.N * st.r * esz + int(lv.sum()) * st.R * 4)
        res[st.name] = {
            "base_us": us["base"],
            "base_GB/s": float(np.mean(byt)) / (us["base"] * 1e-6) / 1e9,
            "base_then_expand_us": us["base"] + us["expand"],
            "fused_us": us["fused"],
            "fused_GB/s": float(np.mean(fbyt)) / (us["fused"] * 1e-6) / 1e9,
            "saved_us": us["base"] + us["expand"] - us["fused"],
        }
    res["how"] = (f"HIP events around runs of one call per layer over {len(use)} rotated "
                  f"layers, {rounds} runs each; LoRA s from the stage's shrink")
    return res


def prefill_base_leg(cfg, host_inputs, delta_graph_us, torch, rounds=5):
    """Context at prefill, beside the headline and not part of it: the base grouped GEMM of
    each stage, one hipBLASLt GEMM (torch.mm) per base expert over that expert's rows already
    gathered (the gather is not timed), on random weights of the stage's shape. This library
    does not build a prefill base GEMM; the leg shows what share of a layer the delta is."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(20240601)
    t = host_inputs[0].topk_ids.reshape(-1)
    loc = (t >= 0) & (t < cfg.E)
    counts = np.bincount(t[loc], minlength=cfg.E)
    starts = np.concatenate([[0], np.cumsum(counts)])
    P = int(counts.sum())
    res = {"what": "base grouped GEMM for context: one torch.mm (hipBLASLt) per base expert "
                   "over its gathered rows, bf16, random weights; not this library's code and "
                   "not part of us_per_layer", "local_pairs": P}
    total = 0.0
    for si, st in enumerate(cfg.stages):
        W = torch.randn(cfg.E, st.N, st.K, device=dev, dtype=torch.bfloat16, generator=g)
        X = torch.randn(P, st.K, device=dev, dtype=torch.bfloat16, generator=g)
        Y = torch.empty(P, st.N, device=dev, dtype=torch.bfloat16)
        # each expert's weight as its own contiguous [K, N] operand (no transposed view)
        Wt = [W[e].t().contiguous() if counts[e] else None for e in range(cfg.E)]
        del W

        def run():
            for e in range(cfg.E):
                if counts[e]:
                    torch.mm(X[starts[e]:starts[e + 1]], Wt[e], out=Y[starts[e]:starts[e + 1]])
        run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(rounds):
            run()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / rounds
        flop = 2.0 * P * st.N * st.K
        res[st.name] = {"us": us, "TFLOP/s": flop / (us * 1e-6) / 1e12,
                        "frac_of_bf16_dense_peak": flop / (us * 1e-6) / 1e12 / 2500.0}
        total += us
        del X, Y, Wt
        torch.cuda.empty_cache()
    res["base_us"] = total
    if delta_graph_us:
        res["delta_us"] = delta_graph_us
        res["base_plus_delta_us"] = total + delta_graph_us
        res["delta_share"] = delta_graph_us / (total + delta_graph_us)
    return res


def kernel_name(cfg, st, kind):
    """The kernel instantiations libmol launches for this stage, as a profiler names them.
    Shrink: rows per work item start at 4 and double while two such items' A rows fit
    32 KiB (at most 32); lanes per row = 256 / rows per item; the weights are held in
    registers when a lane's share of a row fits 8 vectors of 16 bytes. Expand: 16-byte
    vectors per B row = r * element size / 16."""
    esz = 2 if cfg.dtype == "bf16" else 4
    b = "true" if cfg.dtype == "bf16" else "false"
    # from 4096 pairs and 8 pairs per bucket on average (bf16) every block goes to the MFMA
    # kernels and no VALU kernel is launched; the expand also needs r % 32 == 0, r <= 128,
    # R <= 256 and a slice width that is a multiple of 64, and takes the align's plan (the
    # layer passes one) as runs of blocks
    mfma = cfg.dtype == "bf16" and cfg.numel >= 4096 and cfg.numel >= 8 * (cfg.V + 1)
    if kind == "shrink":
        if mfma:
            return f"shrink_mfma_kernel<{2 if st.R > 64 else 1}>"
        lpr = 256 // shrink_rows_per_item(cfg, st)
        held = "true" if st.K * esz // 16 <= 8 * lpr else "false"
        return f"shrink_kernel<{b}, {lpr}, {held}>"
    if (mfma and st.r % 32 == 0 and st.r <= 128 and st.R <= 256
            and (st.N // st.slices) % 64 == 0):
        return f"expand_mfma_run_kernel<{st.r // 32}>"
    return f"expand_kernel<{b}, {st.r * esz // 16}>"


def reference_ctas(grid_m, n, block_n=64):
    """Launch grid of a stage in the reference geometry: one CTA per (M block of the
    worst-case routing buffer, N tile)."""
    return grid_m * -(-n // block_n)


def reference_grid_m(cfg):
    """Blocks of the reference's worst-case routing buffer: every one of the V + 1 buckets
    padded by BLOCK_M - 1 (here the delta grids follow the real pairs instead)."""
    return -(-(cfg.numel + (cfg.V + 1) * (cfg.block_m - 1)) // cfg.block_m)


def code_sha256(sources):
    """SHA-256 of C/HIP source texts with the comments and the layout of whitespace left out:
    a change of wording keeps the hash, any change of the code itself does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for src in sources:
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)  # block comments
        src = re.sub(r"//[^\n]*", " ", src)                # line comments
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def delta_source_sha256():
    """Hash of the delta kernels' code (VALU and MFMA kernels and their device helpers), as
    recorded in the counter summaries."""
    return code_sha256(open(os.path.join(ROOT, "virtual_expert_routed_amd", "csrc", f)).read()
                       for f in ("delta.hip", "delta_mfma.hip", "delta_common.h"))


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` at `workload` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a copy of known size).
    None when there is no summary for this kernel, or the kernel source has changed since
    the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{workload}.md")
    if not os.path.exists(path):
        return None, "no counter summary for this workload"
    text = open(path).read()
    fields = dict(re.findall(r"^(\w+):\s*(.+?)\s*$", text, flags=re.M))
    if fields.get("kernel") != kernel:
        return None, f"counter summary covers {fields.get('kernel')}, not {kernel}"
    if fields.get("kernel_source_sha256") != delta_source_sha256():
        return None, "kernel source changed since the counters were taken"
    return float(fields["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)


def copy_calibration(torch, gib=2, launches=5):
    """An elementwise copy (negation) of `gib` GiB of fp32 into another `gib` GiB, several
    launches back to back: the measured peak for a kernel that reads and writes HBM, and
    the known-size kernel the FETCH_SIZE and WRITE_SIZE counters are scaled by."""
    n = (gib << 30) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    times = []
    for _ in range(launches):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.neg(src, out=dst)
        b.record()
        times.append((a, b))
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in times]
    best = min(us)
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": f"torch.neg fp32 {gib} GiB -> {gib} GiB", "bytes_read": n * 4,
            "bytes_written": n * 4, "launches": launches, "us_best": best,
            "us_median": float(np.median(us)), "GB/s": 2 * n * 4 / (best * 1e-6) / 1e9}


def read_floor(cfg, kernels, grid, layers, torch, reps=20):
    """The read-only streaming probe (libmolcalib.so) at the shapes of the delta's launches:
    for each launch, as many 256-thread workgroups as the kernel has live work items, each
    reading one chunk of (the launch's algorithmic bytes / items) after one dependent index
    load, with no arithmetic and no stores. Every launch of a rotation of `layers` layers reads
    its own random chunks of a 4 GiB buffer, so none is served from the memory-side cache.
    Timed as graph replays: each shape alone (back to back over the layers), and the launches
    of one layer in dependency order (the delta's chain of kernels), per layer."""
    import ctypes
    from virtual_expert_routed_amd import build as hb
    lib = ctypes.CDLL(hb.CALIB_LIB)
    fn = lib.molcal_read_chunks
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    shapes = []
    for k in kernels:
        items = max(1, int(round(grid[k["label"]]["live_blocks_items"])))
        chunk = max(16, int(round(k["bytes"] / items / 16)) * 16)
        shapes.append((k["label"], items, chunk))
    buf_bytes = 4 << 30
    per_layer = sum(n * c for _, n, c in shapes)
    L = min(layers, int(buf_bytes / (1.5 * per_layer)))
    if L < 1:
        return {"skipped": f"one layer's launches read {per_layer / 1e9:.2f} GB, more than "
                           f"the probe's {buf_bytes >> 30} GiB buffer holds with slack"}
    dev = torch.device("cuda")
    buf = torch.full((buf_bytes // 4,), 0x01010101, dtype=torch.int32, device=dev)
    sink = torch.zeros(max(n for _, n, _ in shapes), dtype=torch.int32, device=dev)
    rng = np.random.default_rng(12345)
    idx = []  # idx[l][j]: chunk indices (in units of its chunk size) of launch j of layer l
    off = 0
    for l in range(L):
        row = []
        for _, n, c in shapes:
            region = int(1.5 * n * c) // c  # chunk slots of this launch's own region
            pick = rng.choice(region, size=n, replace=False) + off // c
            row.append(torch.from_numpy(pick.astype(np.int32)).to(dev))
            off += region * c
        idx.append(row)

    def launch(l, j):
        _, n, c = shapes[j]
        rc = fn(buf.data_ptr(), buf_bytes, idx[l][j].data_ptr(), n, c, sink.data_ptr(),
                torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"molcal_read_chunks: {rc}")

    def graph_time(body, per):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                body()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * per)

    res = {"layers": L, "launches": []}
    for j, (label, n, c) in enumerate(shapes):
        us = graph_time(lambda j=j: [launch(l, j) for l in range(L)], L)
        res["launches"].append({"label": label, "workgroups": n, "chunk_bytes": c,
                                "us": us, "GB/s": n * c / (us * 1e-6) / 1e9})
    res["chain_us_per_layer"] = graph_time(
        lambda: [launch(l, j) for l in range(L) for j in range(len(shapes))], L)
    res["chain_bytes"] = per_layer
    res["how"] = ("read-only probe (libmolcalib.so): one 256-thread workgroup per live work "
                  "item, one dependent index load, then its chunk with 16-byte loads; graph "
                  f"replays over {L} layers' disjoint random chunks of a 4 GiB buffer")
    del buf, sink
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the path has no multi-GPU form (asked for "
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
    host_inputs, layers, input_hashes = [], [], []
    for l in range(L):
        inp = inputs.generate(cfg, seed=l)
        input_hashes.append(inputs.sha256(inp))
        base = [inputs.base_out(cfg, si, seed=l) for si in range(len(cfg.stages))]
        layers.append(DeviceLayer(inp, device=dev, outs=base,
                                  topk_weights=inputs.topk_weights(cfg, l)))
        host_inputs.append(inp)
    torch.cuda.synchronize()

    # warm-up (also fills the routing used for the byte model)
    log(f"[bench] warmup {args.warmup} steps")
    for i in range(max(1, args.warmup)):
        layers[i % L].run()
    for dl in layers:   # every layer's routing, whatever the warm-up count
        dl.align()
    torch.cuda.synchronize()
    stats = [layer_stats(dl) for dl in layers]

    def step_body(dl):
        dl.align()
        for si in range(len(cfg.stages)):
            dl.delta(si)

    # A serving engine captures a whole forward pass, all layers, into one graph; likewise
    # the rotation of L layers is one graph here, and single-layer graphs cover a K that
    # is not a multiple of L.
    graph_all, graphs = None, None
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
            graph_all = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph_all, stream=s):
                for dl in layers:
                    step_body(dl)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for _ in range(2):
            graph_all.replay()
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
        for _ in range(K // L):
            graph_all.replay()
        for i in range(K % L):
            graphs[i].replay()
    else:
        for i in range(K):
            step_body(layers[i % L])
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_elapsed = ev0.elapsed_time(ev1) * 1e-3
    # the delta alone (both stages' mol_lora_delta, routing already in place) as graph replays
    # of the rotation: the fused shrink + expand back to back, as a layer runs them
    delta_graph_us = None
    if graphs is not None:
        for dl in layers:
            dl.align()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            g_delta = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_delta, stream=s2):
                for dl in layers:
                    for si in range(len(cfg.stages)):
                        dl.delta(si)
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        g_delta.replay()
        nrep = max(1, K // L)
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        d0.record()
        for _ in range(nrep):
            g_delta.replay()
        d1.record()
        torch.cuda.synchronize()
        delta_graph_us = d0.elapsed_time(d1) * 1e3 / (nrep * L)
        del g_delta

    # spread of the layer time: HIP events around single replays of the rotation graph (or
    # single eager steps), outside the timed region
    dist = []
    nd = max(32, min(64, K // L if graphs is not None else K))
    for i in range(nd):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if graphs is not None:
            graph_all.replay()
        else:
            step_body(layers[i % L])
        e1.record()
        dist.append((e0, e1))
    torch.cuda.synchronize()
    per_layer = np.array([a.elapsed_time(b) * 1e3 / (L if graphs is not None else 1)
                          for a, b in dist])
    # the layers each step used (the rotation restarts after the full-graph replays)
    step_layers = [i % L for i in range(L * (K // L))] + list(range(K % L)) \
        if graphs is not None else [i % L for i in range(K)]

    # ---- per-kernel times: HIP events on the launch stream around runs of L launches of
    # one kernel (one per layer), so each run is timed back to back like the kernels of a
    # step and the event overhead is spread over L launches. Captured graphs cannot hold
    # timing events on ROCm, so this pass launches the same kernels eagerly on the same
    # layers (mol_lora_shrink and mol_lora_expand run the kernels mol_lora_delta
    # enqueues), in dependency order: all aligns, then each stage's shrinks, then its
    # expands. A GPU sleep queued first lets the host enqueue everything ahead of the GPU.
    nst = len(cfg.stages)
    rounds = max(1, min(K, 8 * L) // L)
    launches = [("align", None, lambda dl: dl.align())]
    for si in range(nst):
        launches.append(("shrink", si, lambda dl, si=si: dl.shrink(si)))
        launches.append(("expand", si, lambda dl, si=si: dl.expand(si)))
    # the step after the path (reported beside it, not part of the layer time): the combine
    # of the down stage's rows, and the down expand fused with the combine
    # (the fused form only at decode sizes: it reads B_v per pair, once per token)
    launches.append(("combine", nst - 1, lambda dl: dl.combine()))
    fused_timed = cfg.M <= 1024
    if fused_timed:
        launches.append(("expand_combine", nst - 1, lambda dl: dl.expand_combine()))
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in launches] for _ in range(rounds)]
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
    for r in range(rounds):
        for j, (_, _, fn) in enumerate(launches):
            evs[r][j][0].record()
            for dl in layers:
                fn(dl)
            evs[r][j][1].record()
    torch.cuda.synchronize()

    def per_launch_us(j):
        return float(np.mean([evs[r][j][0].elapsed_time(evs[r][j][1]) for r in range(rounds)])
                     ) * 1e3 / L

    align_us = per_launch_us(0)
    kernels = []
    for j, (kind, si, _) in enumerate(launches[1:], start=1):
        if kind not in ("shrink", "expand"):
            continue
        st = cfg.stages[si]
        fn = shrink_bytes if kind == "shrink" else expand_bytes
        kernels.append({"label": f"{kind} {st.name}", "kernel": kernel_name(cfg, st, kind),
                        "us": per_launch_us(j),
                        "bytes": float(np.mean([fn(cfg, st, s) for s in stats]))})
    stage_b = [float(np.mean([stage_bytes(cfg, st, s) for s in stats])) for st in cfg.stages]

    steps_P = sum(stats[l]["P"] for l in step_layers)
    ms_per_step = elapsed / K * 1e3
    value = steps_P / elapsed
    dom = max(kernels, key=lambda k: k["us"])
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    delta_us = sum(k["us"] for k in kernels)
    delta_bytes = sum(stage_b)
    timing_src = (f"hip-events around runs of {L} back-to-back launches of one kernel (one per "
                  f"layer), {rounds} runs each, eager, queued behind a {spacer_ms:.0f} ms GPU "
                  f"sleep")
    traffic, traffic_src = measured_traffic(cfg.name, dom["kernel"])

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
        "inputs_sha256": input_hashes,
        "us_per_layer": ms_per_step * 1e3,
        "us_per_layer_gpu_events": gpu_elapsed / K * 1e6,
        "us_per_layer_dist": {
            "p10": float(np.percentile(per_layer, 10)),
            "p50": float(np.percentile(per_layer, 50)),
            "p90": float(np.percentile(per_layer, 90)),
            "samples": int(per_layer.size),
            "how": ("HIP events around single replays of the rotation graph, divided by the "
                    "layers in it" if graphs is not None else "HIP events around single steps"),
        },
        "align_us": align_us,
        "pairs_per_layer": float(np.mean([s["P"] for s in stats])),
        "touched_virtual_experts": float(np.mean([s["D"] for s in stats])),
        "kernels": [{"label": k["label"], "kernel": k["kernel"], "us": k["us"],
                     "GB/s": k["bytes"] / (k["us"] * 1e-6) / 1e9} for k in kernels],
        "delta_us": delta_us,
        "grid_workgroups": grid_report(cfg, layers[0].max_blocks, stats),
        "reference_geometry_ctas": {
            f"{kind} {st.name}": reference_ctas(reference_grid_m(cfg), st.R if kind == "shrink"
                                                else st.N // st.slices)
            for st in cfg.stages for kind in ("shrink", "expand")},
        "delta_hbm_frac": delta_bytes / (delta_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "delta_graph_us": delta_graph_us,
        "delta_graph_hbm_frac": (delta_bytes / (delta_graph_us * 1e-6) / 1e9 / HBM_PEAK_GBS
                                 if delta_graph_us else None),
        "kernel_timing": timing_src,
        "roofline": {
            "kernel": f"{dom['kernel']} ({dom['label']})",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_source": traffic_src,
            "bytes_per_launch": dom["bytes"],
            "us_per_launch": dom["us"],
        },
    }
    if cfg.name == configs.N2.name:
        # the pages' own numbers for these stages on this shape (MindLab sglang PR 24: the
        # root-cause passage and the PR body's background): B300, one real model's routing,
        # before their grid fix, which they estimate takes the down expand to ~40 us
        by_label = {k["label"]: k["us"] for k in kernels}
        pages = {"expand down": 160.6, "expand gate_up": 7.5 + 6.8}
        result["pages_comparison"] = {
            "what": ("this library's launch per stage on the pages' decode shape against the "
                     "pages' B300 time for the same stage before their fix (their gate and up "
                     "expands are two launches, 7.5 + 6.8 us; here one two-slice launch); other "
                     "hardware and routing: context, not a target"),
            "pages_down_expand_estimate_after_fix_us": 40.0,
            **{lab: {"pages_us": p, "us": by_label[lab], "pages_over_ours": p / by_label[lab]}
               for lab, p in pages.items()},
        }
    if cfg.M <= 1024:
        result["base_gemm"] = base_gemm_leg(cfg, layers, host_inputs, torch)
    elif cfg.dtype == "bf16":
        log("[bench] base grouped GEMM for context (hipBLASLt per base expert)")
        result["base_gemm"] = prefill_base_leg(cfg, host_inputs, delta_graph_us, torch)
    else:
        result["base_gemm"] = None
    down = cfg.stages[-1]
    n_local = [int(((h.topk_ids >= 0) & (h.topk_ids < cfg.E)).sum()) for h in host_inputs]
    cb = float(np.mean([combine_bytes(cfg, down, n) for n in n_local]))
    fb = float(np.mean([fused_combine_bytes(cfg, down, st_, n)
                        for st_, n in zip(stats, n_local)]))
    comb_us = per_launch_us(2 * nst + 1)
    fused_us = per_launch_us(2 * nst + 2) if fused_timed else None
    down_expand_us = per_launch_us(2 * nst)
    result["combine"] = {
        "what": "router-weighted sum of each token's down-stage rows (not part of us_per_layer)",
        "combine_kernel": "combine_kernel<%s>" % ("true" if cfg.dtype == "bf16" else "false"),
        "combine_us": comb_us,
        "combine_GB/s": cb / (comb_us * 1e-6) / 1e9,
        "down_expand_then_combine_us": down_expand_us + comb_us,
        "fused_kernel": "expand_combine_kernel<%s, %d>" % (
            "true" if cfg.dtype == "bf16" else "false",
            down.r * (2 if cfg.dtype == "bf16" else 4) // 16),
        "fused_expand_combine_us": fused_us,
        "fused_GB/s": fb / (fused_us * 1e-6) / 1e9 if fused_timed else None,
        "fused_hbm_frac": fb / (fused_us * 1e-6) / 1e9 / HBM_PEAK_GBS if fused_timed else None,
    }
    # the achievable peak on this machine: a 2 GiB -> 2 GiB elementwise copy, beside the spec
    cp = copy_calibration(torch)
    result["copy_calibration"] = cp
    result["roofline"]["measured_peak"] = cp["GB/s"]
    result["roofline"]["measured_peak_source"] = cp["kernel"] + " (best of %d)" % cp["launches"]
    result["roofline"]["frac_of_measured_peak"] = achieved / cp["GB/s"]
    result["delta_graph_frac_of_measured_peak"] = (
        delta_bytes / (delta_graph_us * 1e-6) / 1e9 / cp["GB/s"] if delta_graph_us else None)
    if not args.no_floor:
        log("[bench] read-only probe at the delta launches' shapes")
        fl = read_floor(cfg, kernels, result["grid_workgroups"], L, torch)
        if "chain_us_per_layer" in fl and delta_graph_us:
            fl["delta_graph_us_over_chain"] = delta_graph_us / fl["chain_us_per_layer"]
        result["read_floor"] = fl

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
        # the same passes on one thread, over a short sample
        nt = oracle.num_threads()
        oracle.set_num_threads(1)
        t1 = time.perf_counter()
        n1 = 0
        while n1 < 1 or time.perf_counter() - t1 < min(3.0, args.cpu_seconds / 4):
            oracle.run_layer(host_inputs[n1 % L])
            n1 += 1
        el1 = time.perf_counter() - t1
        oracle.set_num_threads(nt)
        cpu_model = ""
        try:
            for ln in open("/proc/cpuinfo"):
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        result["cpu_baseline"] = {
            "value": n_pairs / el, "unit": "pairs/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_layers} whole layer passes of {cfg.name} (layers 0..{L - 1} "
                      f"cycled), fp64 C oracle, {el:.1f} s",
            "us_per_layer": el / n_layers * 1e6,
            "single_thread_us_per_layer": el1 / n1 * 1e6,
            "cpu_model": cpu_model,
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
