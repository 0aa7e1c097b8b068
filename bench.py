"""Benchmark of the routed-expert MXFP4 hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
router logits (fp64) and top-16 selection, the stable bucket by expert, the
grouped SiTU-GLU up-projection (w1, w3), the down-projection (w2) and the
weighted combine. The default workload is one decode token through one
LatentMoE layer whose 896 MXFP4 experts sit in HBM (15.72 GB); each step takes
the next of 64 distinct tokens so that the experts it reads are not the ones
the previous step left in the 256 MB Infinity Cache.

Output: one JSON line (rank 0) with the whole-job throughput, the roofline of
the dominant kernel (its HIP-event time on the stream it runs on) and the CPU
oracle timed on a bounded sample on the host cores.

    python bench.py [--steps K] [--warmup W]
                    [--workload decode_b1|decode_b64|prefill_4096_idot|prefill_4096_exact]
                    [--mfma-decode] [--idot-int8 | --idot-bf16]

The default run (decode_b1) also measures, on the same resident bank:
  other_workloads     short runs of the 64-token EXACT layer (vector and FP4
                      matrix-core forms), the 4096-token IDOT layer (bf16 and
                      int8 matrix-core forms) and the 4096-token EXACT layer on
                      the FP4 matrix cores;
  expert_b1           one expert on one token and the one-matrix product;
  achievable          the sustained matrix-core rates and streaming-read rate
                      (the roofline's achievable denominators);
  launch_costs        a launch, a dependent second launch and an in-launch
                      handoff between workgroups (the bound on one expert);
  block_256[_vector]  the full LatentMoE block at 256 tokens, with the
                      library's default layer form (FP4 matrix cores) and the
                      vector form;
  scale_format        the same product with f32 per-group scales;
  streaming_tier      decode steps with the bank in host memory and an LRU of
                      expert slots in HBM.
Every line carries per-step medians (step_us) and per-stage HIP-event times.
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

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
MFMA_PEAK_I8_TOPS = 5000.0      # MI355X dense int8 matrix, published (tera-ops)
MFMA_PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
MFMA_PEAK_FP4_TFLOPS = 10100.0  # MI355X dense fp4 matrix, published
MFMA_PEAK_F64_TFLOPS = 78.6     # MI355X fp64 matrix, published
N_ROT = 64                 # distinct tokens the decode steps cycle through


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_b1", choices=["decode_b1", "decode_b64", "prefill_4096_idot", "prefill_4096_exact"])
    ap.add_argument("--idot-int8", action="store_true",
                    help="IDOT workloads: run the group dots on the int8 matrix cores (same results; without it the "
                         "library's default, the bf16 matrix cores)")
    ap.add_argument("--idot-bf16", action="store_true",
                    help="IDOT workloads: the bf16 matrix-core form, named (the default)")
    ap.add_argument("--mfma-decode", action="store_true",
                    help="EXACT workloads and the block: the expert products on the FP4 matrix cores (x and h as "
                         "e2m1 pieces) whatever the token count")
    ap.add_argument("--vector-decode", action="store_true",
                    help="EXACT workloads and the block: the vector kernels whatever the token count (without "
                         "either flag: the library's default, vector for one token, FP4 matrix cores for more)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="decode_b1 only: skip the short runs of the 64-token and 4096-token workloads")
    ap.add_argument("--eager", action="store_true", help="launch every kernel from Python instead of HIP graphs")
    ap.add_argument("--stream-steps", type=int, default=40,
                    help="decode steps per cache size in the streaming-tier measurement")
    ap.add_argument("--achievable-only", action="store_true",
                    help="only measure the matrix-core rates and a streaming read (the achievable peaks) and exit")
    ap.add_argument("--expert-only", action="store_true",
                    help="only time one expert on one token and the batch-1 product (for profiling) and exit")
    ap.add_argument("--stream-only", action="store_true",
                    help="only the expert streaming tier (bank in host memory, LRU of slots in HBM)")
    ap.add_argument("--block-only", action="store_true",
                    help="only time the 256-token LatentMoE block (for profiling) and exit")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="only copy a GIB-sized buffer 5 times (a plain copy of known size, for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--bank-experts", type=int, default=0,
                    help="diagnostic: a bank (and router) of this many experts instead of 896, to compare a "
                         "kernel's rate on a smaller allocation (not a configuration of the method)")
    args = ap.parse_args()
    if args.idot_int8 and args.idot_bf16:
        ap.error("--idot-int8 and --idot-bf16 name different forms")
    return args


def expert_bytes(latent, inter):
    """Bytes of one expert's w1 + w3 (up) and of its w2 (down)."""
    up = 2 * inter * (latent // 2 + latent // 32)
    dn = latent * (inter // 2 + inter // 32)
    return up, dn


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs the path on a single MI355X and has no "
              "multi-GPU mode; run it with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    if args.copy_calibration > 0:
        return copy_calibration(torch, args.copy_calibration)

    import mxfp4_moe_expert_amd as k3g
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    k3g.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    L, I, E = synth.LATENT, synth.INTER, (args.bank_experts or synth.N_EXPERTS)
    seed_bank = synth.SEED_BASE + 1
    t0 = time.time()
    src = lambda e: synth.expert(seed_bank, e)  # noqa: E731
    bankt, bank = k3g.pack_bank(src, E, L, I)
    print(f"# setup {time.time() - t0:.1f}s: bank {bankt.numel() / 1e9:.2f} GB", file=sys.stderr, flush=True)

    ctx = dict(torch=torch, k3g=k3g, synth=synth, dev=dev, bank=bank, seed_bank=seed_bank, eager=args.eager,
               n_experts=E)
    form_arg = "mfma" if args.mfma_decode else "vector" if args.vector_decode else None
    if args.achievable_only:
        print(json.dumps({"achievable": run_achievable(ctx)}), flush=True)
        return
    if args.expert_only:
        print(json.dumps({"expert_b1": run_expert(ctx, bankt)}), flush=True)
        return
    if args.stream_only:
        print(json.dumps({"streaming_tier": run_stream(ctx, bankt, configs=((64, 0.1), (256, 0.1), (256, 0.01)),
                                                       steps=args.stream_steps)}), flush=True)
        return
    if args.block_only:
        print(json.dumps({"block_256": run_block(ctx, bank, form=form_arg)}), flush=True)
        return
    result, host = run_workload(ctx, args.workload, args.steps, args.warmup, args.idot_int8, form_arg)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, src, *host)
    if args.workload == "decode_b1" and not args.no_secondary:
        # the other configurations on the same resident bank, shorter runs (not the headline)
        others = []
        cpu_lines = {}
        for wl, steps, warm, int8, p, fm in (("decode_b1", 100, 10, False, 0.9, None),
                                             ("decode_b64", 20, 3, False, 0.0, None),
                                             ("decode_b64", 20, 3, False, 0.0, "vector"),
                                             ("prefill_4096_idot", 10, 2, False, 0.0, None),
                                             ("prefill_4096_idot", 10, 2, True, 0.0, None),
                                             ("prefill_4096_exact", 5, 1, False, 0.0, None)):
            r, h = run_workload(ctx, wl, steps, warm, int8, form_name=fm, top_p=p)
            rec = {k: r[k] for k in ("config", "ms_per_step", "value", "unit", "tokens_per_s", "step_us",
                                     "stage_us", "decode", "roofline", "steps", "warmup")}
            if not args.no_cpu_baseline and wl != "decode_b1":
                key = (wl, h[-1])  # the oracle does not depend on the GPU form
                if key not in cpu_lines:
                    cpu_lines[key] = cpu_baseline(args, src, *h, budget=args.cpu_seconds / 2)
                rec["cpu_baseline"] = cpu_lines[key]
            others.append(rec)
        result["other_workloads"] = others
        # one expert on one token, and the batch-1 product on one w1
        result["expert_b1"] = run_expert(ctx, bankt)
        if not args.no_cpu_baseline:
            result["expert_b1"]["cpu_baseline"] = cpu_expert(args, ctx, src)
        # the achievable denominators: matrix-core rates and a streaming read
        result["achievable"] = run_achievable(ctx, launch_bytes=result["roofline"]["algorithmic_bytes_per_launch"])
        ach = result["achievable"]["hbm_read"]["GBps"]
        result["roofline"]["achievable_peak"] = ach
        result["roofline"]["frac_of_achievable"] = round(result["roofline"]["achieved"] / ach, 4)
        ach_l = result["achievable"]["hbm_read_at_launch_size"]["GBps"]
        result["roofline"]["achievable_at_launch_size"] = ach_l
        result["roofline"]["frac_of_achievable_at_launch_size"] = round(result["roofline"]["achieved"] / ach_l, 4)
        # what a launch and a handoff between workgroups cost (the bound on one expert)
        result["launch_costs"] = run_launch_costs(ctx)
        # the full LatentMoE block at 256 tokens, the routed layer in both forms
        result["block_256"] = run_block(ctx, bank)  # the library's default form (FP4 matrix-core layer)
        if not args.no_cpu_baseline:
            result["block_256"]["cpu_baseline"] = cpu_block(args, ctx, src)
        result["block_256_vector"] = run_block(ctx, bank, form="vector")
        # the Vulkan-tier scale format: the same product with f32 per-group scales
        result["scale_format"] = run_scale_format(ctx)
        # the expert streaming tier: the bank in pinned host memory, an LRU of slots in HBM
        result["streaming_tier"] = run_stream(ctx, bankt, configs=((64, 0.1), (256, 0.1), (256, 0.01)),
                                              steps=args.stream_steps)
    print(json.dumps(result), flush=True)


def run_workload(ctx, workload, steps, warmup, idot_int8, form_name=None, top_p=0.0):
    """Measure one workload on the resident bank. Returns the result record and
    what the CPU baseline needs (the same inputs)."""
    torch, k3g, synth, dev, bank = ctx["torch"], ctx["k3g"], ctx["synth"], ctx["dev"], ctx["bank"]
    L, I, E, K = synth.LATENT, synth.INTER, ctx["n_experts"], synth.TOP_K
    wl_seed, T, bias_range, mode_name = synth.WORKLOADS[workload]
    mode = k3g.IDOT if mode_name == "idot" else k3g.EXACT
    form = 0
    if mode == k3g.IDOT:  # named either way (the bf16 form is the library's default)
        form = k3g.IDOT_INT8 if idot_int8 else k3g.IDOT_BF16
    if mode == k3g.EXACT:  # None: the library's default (vector for one token, FP4 matrix cores for more)
        form = {None: 0, "vector": k3g.DECODE_VECTOR, "mfma": k3g.DECODE_MFMA}[form_name]

    W, b = synth.router(wl_seed, E, L, bias_range)
    Wd = torch.from_numpy(W).to(dev)
    bd = torch.from_numpy(b).to(dev)
    n_rot = N_ROT if T == 1 else 4
    xs_host = [synth.activations(wl_seed, T, L, key=r) for r in range(n_rot)]
    xs = [torch.from_numpy(x).to(dev) for x in xs_host]

    # per input batch r: its own routing, workspaces and output, so that any
    # stage can be replayed over all batches
    idx = [torch.empty((T, K), dtype=torch.int32, device=dev) for _ in range(n_rot)]
    wts = [torch.empty((T, K), dtype=torch.float32, device=dev) for _ in range(n_rot)]
    ys = [torch.empty((T, L), dtype=torch.float32, device=dev) for _ in range(n_rot)]
    ws_r = [k3g.workspace(k3g.OP_MOE_ROUTE, k3g.shape(n_tokens=T, n_experts=E)) for _ in range(n_rot)]
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=L, inter=I, mode=mode | form)
    ws = [k3g.workspace(k3g.OP_MOE_LAYER, sh) for _ in range(n_rot)]

    # the FP4 matrix-core form (QUANT_X splits x into pieces): asked for, or the default here
    f4 = bool(k3g.workspace_layout(k3g.OP_MOE_LAYER, sh)["xp"])
    stages = [("route", None), ("bucket", k3g.STAGE_BUCKET)]
    if mode == k3g.IDOT or f4:
        stages.append(("quant_x", k3g.STAGE_QUANT_X))
    stages.append(("up", k3g.STAGE_UP))
    if mode == k3g.IDOT or f4:
        stages.append(("quant_h", k3g.STAGE_QUANT_H))
    stages += [("down", k3g.STAGE_DOWN), ("combine", k3g.STAGE_COMBINE)]

    ws_by_mode = {mode | form: ws}
    if f4 and form == 0:  # name the form the default took, so the per-stage calls below see the same one
        form = k3g.DECODE_MFMA
        ws_by_mode = {mode | form: ws}

    def stage(r, st, m=mode | form):
        if st is None:
            if top_p:
                k3g.k3g_moe_route_topp(idx[r], wts[r], xs[r], Wd, bd, K, top_p, ws_r[r])
            else:
                k3g.k3g_moe_route(idx[r], wts[r], xs[r], Wd, bd, K, ws_r[r])
        else:
            if m not in ws_by_mode:  # another decode form: a workspace of its own size
                shm = k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=L, inter=I, mode=m)
                ws_by_mode[m] = [k3g.workspace(k3g.OP_MOE_LAYER, shm) for _ in range(n_rot)]
            k3g.k3g_moe_layer_stage(st, ys[r], xs[r], idx[r], wts[r], bank, m, ws_by_mode[m][r])

    def step(r):
        for _, st in stages:
            stage(r, st)

    # eager warm-up (also fills the library's per-device checks before capture)
    for r in range(n_rot):
        step(r)
    torch.cuda.synchronize()

    # one HIP graph per input batch holding the whole step
    graphs = []
    if not ctx["eager"]:
        for r in range(n_rot):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i):
        if graphs:
            graphs[i % n_rot].replay()
        else:
            step(i % n_rot)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, host clock between two device syncs
    t_start = time.perf_counter()
    for i in range(steps):
        run(warmup + i)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_per_step = 1e3 * t_total / steps

    # the distribution of single steps (after the timed region): HIP events
    # around each of up to 100 steps
    stream = torch.cuda.current_stream()
    n_single = min(100, max(steps, 10))
    single = []
    for i in range(n_single):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(i)
        e1.record(stream)
        single.append((e0, e1))
    torch.cuda.synchronize()
    single_us = np.array([a.elapsed_time(b) * 1e3 for a, b in single])

    # per-kernel times: each stage replayed over every input batch inside one
    # graph, bracketed by HIP events on the stream it runs on; the average
    # launch time is the elapsed time over the number of launches
    reps = 3

    def time_stage(st, m):
        for r in range(n_rot):  # eager once first: earlier stages' results, and workspaces allocated outside capture
            for _, s0 in stages:
                if st is not None and s0 is not None and s0 < st:
                    stage(r, s0, m)
            stage(r, st, m)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(n_rot):
                stage(r, st, m)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * n_rot)

    # stages that enqueue nothing in this form are reported as null, not timed:
    # one EXACT token ranks its route entries inside the up kernel (no bucket
    # launch), and the FP4 matrix-core up kernel writes h's pieces itself
    empty = set()
    if T == 1 and mode == k3g.EXACT:
        empty.add("bucket")
    if f4 or mode == k3g.IDOT:  # these up kernels write the down product's operand themselves
        empty.add("quant_h")
    stage_ms = {name: (None if name in empty else time_stage(st, mode | form)) for name, st in stages}
    # the same products in the other decode forms: the LDS byte-pair table, and the
    # FP4 matrix cores (x split into pieces first) or the vector convert
    lut_ms, alt_ms = {}, {}
    if mode == k3g.EXACT and T == 1:
        lut_ms = {name: time_stage(st, mode | k3g.DECODE_LUT) for name, st in stages if name in ("up", "down")}
        alt = mode | k3g.DECODE_VECTOR if f4 else mode | k3g.DECODE_MFMA
        alt_ms = {name: time_stage(st, alt) for name, st in
                  [("quant_x", k3g.STAGE_QUANT_X), ("up", k3g.STAGE_UP), ("down", k3g.STAGE_DOWN)]
                  if f4 is False or name != "quant_x"}
    timing = (f"step: {len(graphs) and 'HIP graph per step' or 'eager'} replay; stages: HIP events around a graph "
              f"of {n_rot} launches of the stage, {reps} replays")

    # distinct experts per step (one token: top_k; more tokens, or a K3_TOPP cut:
    # counted from the routing, dropped entries excluded)
    counts = None
    if T > 1 or top_p:
        cnt = []
        for r in range(n_rot):
            ids = idx[r].cpu().numpy()
            cnt.append(len(np.unique(ids[ids >= 0])))
        counts = float(np.mean(cnt))
    n_exp = float(K) if counts is None else counts
    P = T * K if not top_p else int(sum(int((idx[r] >= 0).sum()) for r in range(n_rot)) / n_rot)
    up_b, dn_b = expert_bytes(L, I)
    router_b = E * L * 4 + E * 4
    alg_bytes = n_exp * (up_b + dn_b) + router_b + 2 * T * L * 4
    up_alg = n_exp * up_b + T * L * 4 + P * I * 4       # weights once, x in, h out
    if mode == k3g.IDOT:  # int8 x and its scales in; h out quantised (int8, or bf16 in that form) with its scales
        up_alg = n_exp * up_b + T * L + T * (L // 32) * 4 + P * I * (2 if form == k3g.IDOT_BF16 else 1) + P * (I // 32) * 4

    # the tag of this form in the names of the committed counter summaries
    form_tag = ("fp4_mfma" if f4 else "bf16" if form == k3g.IDOT_BF16 else
                "vector" if (mode == k3g.EXACT and T > 1) else "")
    gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
    tok_s = T / (ms_per_step * 1e-3)
    up_gbs = up_alg / (stage_ms["up"] * 1e-3) / 1e9
    roof = {
        "kernel": "moe_up (w1, w3 and SiTU for every selected expert)",
        "bound": "hbm",
        "achieved": round(up_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(up_gbs / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(workload, "moe_up", form_tag),
        "algorithmic_bytes_per_launch": int(up_alg),
    }
    if f4:
        # the FP4 matrix-core work the up kernel issues: every pair's w1 and w3
        # rows against its 16 pieces of x (2 ops per multiply-add)
        f4_ops = 2.0 * P * 2 * I * L * 16
        f4_t = f4_ops / (stage_ms["up"] * 1e-3) / 1e12
        roof["mfma_fp4_achieved_TFLOPs"] = round(f4_t, 1)
        roof["mfma_fp4_frac"] = round(f4_t / MFMA_PEAK_FP4_TFLOPS, 4)
    if mode == k3g.IDOT:
        # matrix-core work of the up kernel: 2 ops per multiply-add, w1 and w3 rows, every pair
        up_ops = 2.0 * P * 2 * I * L
        bf16 = form == k3g.IDOT_BF16
        peak = MFMA_PEAK_BF16_TFLOPS if bf16 else MFMA_PEAK_I8_TOPS
        tops = up_ops / (stage_ms["up"] * 1e-3) / 1e12
        roof = {
            "kernel": "moe_up (IDOT group dots of w1 and w3 for every pair, SiTU)",
            "bound": "mfma",
            "achieved": round(tops, 1),
            "peak": peak,
            "unit": "TFLOP/s",
            "ops": "bf16 multiply-adds x 2 (exact int8 values)" if bf16 else "int8 multiply-adds x 2",
            "frac": round(tops / peak, 4),
            "traffic": measured_traffic(workload, "moe_up", form_tag),
            "algorithmic_ops_per_launch": up_ops,
            "hbm_achieved_GBps": round(up_gbs, 1),
            "hbm_frac": round(up_gbs / HBM_PEAK_GBS, 4),
        }

    result = {
        "metric": "MXFP4 expert GEMV HBM GB/s (batch 1); MoE-layer tokens/s at 4096 tokens",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if mode == k3g.EXACT else "i8",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "tokens_per_step": T,
            "experts": E, "top_k": K, "latent": L, "inter": I,
            "mode": mode_name + ("+bf16-mfma" if form == k3g.IDOT_BF16 else "+int8-mfma" if form == k3g.IDOT_INT8
                                 else "+fp4-mfma" if f4 else ""),
            "distinct_experts_per_step": n_exp,
            "top_p": top_p,
            "algorithmic_bytes_per_step": int(alg_bytes),
            "seed_bank": ctx["seed_bank"], "seed_workload": wl_seed,
        },
        "tokens_per_s": round(tok_s, 1),
        "step_us": {"n": int(n_single), "median": round(float(np.median(single_us)), 2),
                    "best": round(float(single_us.min()), 2), "worst": round(float(single_us.max()), 2),
                    "timing": "HIP events around each step, back to back"},
        "stage_us": {k: (None if v is None else round(v * 1e3, 2)) for k, v in stage_ms.items()},
        "decode": ("gfx950 FP4 MFMA on the stored nibbles, x and h as 16 e2m1 pieces" if f4 else
                   "gfx950 FP4->FP32 convert" if mode == k3g.EXACT else
                   "bf16 MFMA on exact int8 values" if form == k3g.IDOT_BF16 else "int8 MFMA"),
        ("stage_us_vector_cvt_decode" if f4 else "stage_us_fp4_mfma_decode"):
            {k: round(v * 1e3, 2) for k, v in alt_ms.items()},
        "stage_us_lds_lut_decode": {k: round(v * 1e3, 2) for k, v in lut_ms.items()},
        "timing": timing,
        "roofline": roof,
    }
    # release this workload's device memory before the next one
    del graphs, ws, ws_r, ws_by_mode, idx, wts, ys, xs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result, (xs_host, W, b, alg_bytes, T, mode)


def measured_traffic(workload, kernel, form=""):
    """HBM bytes per launch (read + write) of `kernel` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary `profiles/<workload>[_<form>]_traffic.json`,
    scaled by the copy calibration it records; None when no summary exists or
    the kernel sources it lists have changed since it was taken."""
    import hashlib

    name = f"{workload}_{form}_traffic.json" if form else f"{workload}_traffic.json"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    csrc = os.path.join(ROOT, "mxfp4_moe_expert_amd", "csrc")
    srcs = doc.get("sources", ["gemv.hip", "k3g_common.h"])
    sha = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in srcs)).hexdigest()
    if sha != doc.get("source_sha256") or kernel not in doc.get("kernels", {}):
        return None
    k = doc["kernels"][kernel]
    return int(k["fetch_bytes"] + k["write_bytes"])


def run_block(ctx, bank, reps=10, form=None):
    """The full LatentMoE block on 256 tokens (route on the 7168-wide hidden
    state, bf16 down-projection, the routed layer on the resident bank, RMSNorm,
    bf16 up-projection, two bf16 shared SiTU-GLU experts of 6144): HIP events
    around `reps` calls, and the dense parts' matrix work as a rate."""
    torch, k3g, synth, dev = ctx["torch"], ctx["k3g"], ctx["synth"], ctx["dev"]
    seed, T, bias_range, _ = synth.WORKLOADS["block_256"]
    # form None: the library's default (the FP4 matrix-core layer at 256 tokens)
    mode = k3g.EXACT | {None: 0, "vector": k3g.DECODE_VECTOR, "mfma": k3g.DECODE_MFMA}[form]
    H, Lt, SI, E, K = synth.HIDDEN, synth.LATENT, synth.SHARED_INTER, synth.N_EXPERTS, synth.TOP_K
    dense = {k: torch.from_numpy(v).to(dev) for k, v in synth.block_dense(seed).items()}
    W, b = synth.router(seed, E, H, bias_range)
    x = torch.from_numpy(synth.activations(seed, T, H)).to(dev)
    w = k3g.block_struct(torch.from_numpy(W).to(dev), torch.from_numpy(b).to(dev), dense["w_down"], dense["w_up"],
                         dense["gamma"], [dense[f"sh_w1_{s}"] for s in range(2)],
                         [dense[f"sh_w3_{s}"] for s in range(2)], [dense[f"sh_w2_{s}"] for s in range(2)], bank)
    sh = k3g.shape(n_tokens=T, top_k=K, n_experts=E, latent=Lt, inter=synth.INTER, hidden=H, sh_inter=SI,
                   mode=mode)
    ws = k3g.workspace(k3g.OP_LATENT_BLOCK, sh)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    k3g.k3g_latent_moe_block(out, x, w, K, mode, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        k3g.k3g_latent_moe_block(out, x, w, K, mode, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # the routed layer's distinct experts (from the routing the block wrote)
    L = k3g.workspace_layout(k3g.OP_LATENT_BLOCK, sh)
    idx = ws[L["idx"]: L["idx"] + 4 * T * K].view(torch.int32).cpu().numpy()
    distinct = int(len(set(idx.tolist()) - {-1}))
    # dense matrix work: down, up, and per shared expert w1, w3 and w2 (2 flops per product)
    flops = 2.0 * T * (2 * H * Lt + 2 * 3 * H * SI)
    out_d = {"tokens": T, "layer": "vector" if form == "vector" else "fp4-mfma",
             "ms_per_block": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
             "distinct_experts": distinct,
             "dense_flops": flops, "dense_TFLOPs_if_all_time": round(flops / (ms * 1e-3) / 1e12, 1)}
    del dense, ws, out, x
    torch.cuda.empty_cache()
    return out_d


def run_expert(ctx, bankt, n_rot=64, reps=5):
    """One SiTU-GLU expert on one token (k3g_expert_glu: 17,547,264 B of
    weights + x and y), and the batch-1 product on one w1 (k3g_mxfp4_gemv,
    3072 x 3584). Each call takes the next of n_rot experts spread over the
    bank (1.12 GB, past the 256 MB Infinity Cache). Back to back: a HIP graph
    of n_rot calls, HIP events around `reps` replays. Per launch: HIP events
    around each call alone, the device idle before it."""
    torch, k3g, synth, dev = ctx["torch"], ctx["k3g"], ctx["synth"], ctx["dev"]
    L, I, E = synth.LATENT, synth.INTER, synth.N_EXPERTS
    off, stride = k3g.bank_layout(L, I)
    shapes = {"w1p": (I, L // 2), "w1s": (I, L // 32), "w3p": (I, L // 2), "w3s": (I, L // 32),
              "w2p": (L, I // 2), "w2s": (L, I // 32)}
    keys = ("w1p", "w1s", "w3p", "w3s", "w2p", "w2s")
    experts = []
    for i in range(n_rot):
        e = (i * E) // n_rot
        base = e * stride
        experts.append({k: bankt[base + off[j]: base + off[j] + shapes[k][0] * shapes[k][1]].view(*shapes[k])
                        for j, k in enumerate(keys)})
    x = torch.from_numpy(synth.activations(ctx["seed_bank"], 1, L)[0]).to(dev)
    y = torch.empty(L, dtype=torch.float32, device=dev)
    yg = torch.empty(I, dtype=torch.float32, device=dev)
    ws = k3g.workspace(k3g.OP_EXPERT_GLU, k3g.shape(n_tokens=1, top_k=1, n_experts=1, latent=L, inter=I,
                                                     mode=k3g.EXACT))
    stream = torch.cuda.current_stream()

    def glu(i):
        k3g.k3g_expert_glu(y, x, experts[i % n_rot], k3g.EXACT, ws)

    def gemv(i):
        ex = experts[i % n_rot]
        k3g.k3g_mxfp4_gemv(yg, x, ex["w1p"], ex["w1s"])

    def graph_us(fn):
        for i in range(n_rot):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_rot):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * n_rot)

    def launch_us(fn):
        ts = []
        for i in range(n_rot):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    up_b, dn_b = expert_bytes(L, I)
    glu_bytes = up_b + dn_b + 2 * L * 4
    gemv_bytes = up_b // 2 + L * 4 + I * 4
    out = {"experts_rotated": n_rot, "timing": "graph: HIP events around replays of a graph of one call per "
           "expert; per launch: median over the experts of HIP events around one call on an idle device"}
    for name, fn, nbytes in (("expert_glu", glu, glu_bytes), ("gemv_w1", gemv, gemv_bytes)):
        tg, tl = graph_us(fn), launch_us(fn)
        out[name] = {"bytes": int(nbytes), "graph_us": round(tg, 2), "graph_GBps": round(nbytes / tg / 1e3, 1),
                     "graph_hbm_frac": round(nbytes / tg / 1e3 / HBM_PEAK_GBS, 4),
                     "launch_us": round(tl, 2), "launch_GBps": round(nbytes / tl / 1e3, 1)}
    del experts, ws
    torch.cuda.empty_cache()
    return out


def run_achievable(ctx, reps=3, launch_bytes=None):
    """What this chip sustains, beside the datasheet peaks: back-to-back matrix
    products of each kind the path uses (no memory traffic), and one streaming
    read of a 4 GiB buffer; HIP events around `reps` launches after a warm-up.
    With `launch_bytes`, also the same read cut into launches of that size (a
    kernel's bytes per launch), each launch reading the next slice of the 4 GiB
    buffer, so no slice is still in the 256 MB Infinity Cache when read again:
    the rate one launch of that size can reach, ramp-up and tail included."""
    torch, k3g = ctx["torch"], ctx["k3g"]
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1, dtype=torch.int32, device=ctx["dev"])
    products = 2048 * 4 * 4  # workgroups x wavefronts x independent products per round
    kinds = {  # kind: (name, ops per instruction, rounds per launch, published dense peak in T(FL)OP/s)
        0: ("int8", 2 * 32 * 32 * 32, 5000, MFMA_PEAK_I8_TOPS),
        1: ("bf16", 2 * 16 * 16 * 32, 10000, MFMA_PEAK_BF16_TFLOPS),
        2: ("fp4", 2 * 16 * 16 * 128, 10000, MFMA_PEAK_FP4_TFLOPS),
        3: ("fp64", 2 * 16 * 16 * 4, 2500, MFMA_PEAK_F64_TFLOPS),
    }

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    out = {"timing": f"HIP events around {reps} launches after one warm-up launch", "matrix": {}}
    for kind, (name, ops, rounds, peak) in kinds.items():
        t = timed(lambda: k3g.k3g_probe_mfma_rate(kind, rounds, sink))
        rate = products * rounds * ops / t / 1e12
        out["matrix"][name] = {"achieved_TOPs": round(rate, 1), "peak": peak, "frac": round(rate / peak, 4)}
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=ctx["dev"])
    t = timed(lambda: k3g.k3g_probe_read_rate(buf, sink))
    gbs = buf.numel() / t / 1e9
    out["hbm_read"] = {"bytes": buf.numel(), "GBps": round(gbs, 1), "peak": HBM_PEAK_GBS,
                       "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if launch_bytes:
        size = int(launch_bytes) // 16 * 16
        slices = [buf[i * size:(i + 1) * size] for i in range(buf.numel() // size)]
        t = timed(lambda: [k3g.k3g_probe_read_rate(b, sink) for b in slices]) / len(slices)
        out["hbm_read_at_launch_size"] = {"bytes": size, "slices": len(slices), "launch_us": round(t * 1e6, 2),
                                          "GBps": round(size / t / 1e9, 1)}
    del buf
    torch.cuda.empty_cache()
    return out


def run_launch_costs(ctx, launches=64, reps=5):
    """Per launch, back to back in a HIP graph of `launches` calls (HIP events
    around `reps` replays): a grid of n one-wavefront workgroups that each store
    one value (mode 0), the same followed by a dependent one-workgroup launch
    that sums them (mode 1), and the sum done in the same launch by the
    workgroup that counts last on a device counter after an agent-scope release
    by every workgroup (mode 2). Results are checked against the exact sum."""
    torch, k3g, dev = ctx["torch"], ctx["k3g"], ctx["dev"]
    stream = torch.cuda.current_stream()
    out = {"timing": f"HIP events around {reps} replays of a graph of {launches} calls"}
    for n in (64, 256, 896):
        buf = torch.zeros(n + 1, dtype=torch.float32, device=dev)
        cnt = torch.zeros(1, dtype=torch.int32, device=dev)
        want = 0.5 * n * (n - 1) / 2
        rec = {}
        for mode, name in ((0, "one_launch_us"), (1, "two_dependent_launches_us"), (2, "one_launch_last_arriver_us")):
            k3g.k3g_probe_handoff(mode, buf, cnt)
            torch.cuda.synchronize()
            if mode:
                assert abs(float(buf[n]) - want) <= 1e-6 * want + 1e-6, (mode, n, float(buf[n]), want)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(launches):
                    k3g.k3g_probe_handoff(mode, buf, cnt)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            rec[name] = round(e0.elapsed_time(e1) * 1e3 / (reps * launches), 2)
        out[f"workgroups_{n}"] = rec
    return out


def run_scale_format(ctx, n_mat=8, launches=64):
    """The batch-1 product on 16 experts' w1+w3 stacked (49,152 x 3,584), with
    ue8m0 scales and with the scales expanded to f32 at upload (the pages'
    Vulkan-tier format): time per launch (HIP events around `launches`
    launches cycling over n_mat distinct matrices, so no launch finds its
    matrix in the Infinity Cache) and algorithmic bytes per second."""
    torch, k3g, dev = ctx["torch"], ctx["k3g"], ctx["dev"]
    rows, n_in = 16 * 3072, 3584
    g = torch.Generator(device=dev).manual_seed(0x4B33)
    pk = [torch.randint(0, 256, (rows, n_in // 2), dtype=torch.uint8, device=dev, generator=g) for _ in range(n_mat)]
    s8 = [torch.randint(118, 133, (rows, n_in // 32), dtype=torch.uint8, device=dev, generator=g)
          for _ in range(n_mat)]
    s32 = [torch.empty((rows, n_in // 32), dtype=torch.float32, device=dev) for _ in range(n_mat)]
    for a, b in zip(s8, s32):
        k3g.k3g_mxfp4_scales_to_f32(b, a)
    x = torch.randn(n_in, dtype=torch.float32, device=dev, generator=g)
    ys = [torch.empty(rows, dtype=torch.float32, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream()

    def timed(fn):
        for i in range(n_mat):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(launches):
            fn(i % n_mat)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / launches

    us8 = timed(lambda i: k3g.k3g_mxfp4_gemv(ys[0], x, pk[i], s8[i]))
    us32 = timed(lambda i: k3g.k3g_mxfp4_gemv_f32s(ys[1], x, pk[i], s32[i]))
    same = bool(torch.equal(ys[0], ys[1]))
    b8 = rows * (n_in // 2 + n_in // 32) + 4 * (n_in + rows)
    b32 = rows * (n_in // 2 + 4 * (n_in // 32)) + 4 * (n_in + rows)
    out = {"matrix": f"{rows}x{n_in}", "ue8m0_us": round(us8, 2), "ue8m0_GBps": round(b8 / us8 / 1e3, 1),
           "f32_us": round(us32, 2), "f32_GBps": round(b32 / us32 / 1e3, 1),
           "bytes_ue8m0": b8, "bytes_f32": b32, "results_identical": same}
    del pk, s8, s32, ys
    torch.cuda.empty_cache()
    return out


def run_stream(ctx, bankt, configs, steps):
    """Decode with the 896-expert bank in pinned host memory and an LRU of n
    slots in HBM (k3g_cache): each step routes on the GPU, brings the 16 ids to
    the host, plans, copies the misses host -> HBM on a copy stream and runs the
    layer on the slots. configs: (slots, router bias range): 0.1 is the decode
    workload's router (the bias makes some experts hot), 0.01 near-flat use
    (the pages' trained router is balanced to flat use). Host clock around
    `steps` steps after 8 warm-up steps; also the bare pinned host -> HBM copy
    rate of one expert (17.5 MB) at a time. Each configuration runs twice from
    an empty cache with the same tokens: the layer after all of the step's
    copies (k3g_cache_prepare, then k3g_moe_layer), and the pipelined step
    (k3g_cache_decode_step: the resident experts' products during the first
    copy, each copied expert's as soon as its copy lands)."""
    torch, k3g, synth, dev, bank = ctx["torch"], ctx["k3g"], ctx["synth"], ctx["dev"], ctx["bank"]
    L, I, E, K = synth.LATENT, synth.INTER, synth.N_EXPERTS, synth.TOP_K
    off, stride = k3g.bank_layout(L, I)
    host = torch.empty(E * stride, dtype=torch.uint8, pin_memory=True)
    host.copy_(bankt[:E * stride])
    wl_seed = synth.WORKLOADS["decode_b1"][0]
    n_rot = 512
    xs = [torch.from_numpy(synth.activations(wl_seed, 1, L, key=1000 + r)).to(dev) for r in range(n_rot)]
    idx = torch.empty((1, K), dtype=torch.int32, device=dev)
    wts = torch.empty((1, K), dtype=torch.float32, device=dev)
    idx_slot = torch.empty((1, K), dtype=torch.int32, device=dev)
    y = torch.empty((1, L), dtype=torch.float32, device=dev)
    ws_r = k3g.workspace(k3g.OP_MOE_ROUTE, k3g.shape(n_tokens=1, n_experts=E))
    copy_stream = torch.cuda.Stream()
    # bare copy rate: one expert per copy, 64 copies
    dst = torch.empty(stride, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(64):
        dst.copy_(host[(i % E) * stride:(i % E + 1) * stride], non_blocking=True)
    torch.cuda.synchronize()
    bare = 64 * stride / (time.perf_counter() - t0) / 1e9
    out = {"host_bank_bytes": E * stride, "bare_copy_GBps": round(bare, 2),
           "pages_nvme_GBps": 6.3, "note": "host clock, steps include the idx round trip to the host"}
    runs = []
    for n_slots, bias_range in configs:
        W, b = synth.router(wl_seed, E, L, bias_range)
        Wd, bd = torch.from_numpy(W).to(dev), torch.from_numpy(b).to(dev)
        arena_t = torch.empty(n_slots * stride, dtype=torch.uint8, device=dev)
        arena = k3g.bank_struct(arena_t, n_slots, L, I, off, stride)
        sh = k3g.shape(n_tokens=1, top_k=K, n_experts=n_slots, latent=L, inter=I, mode=k3g.EXACT)
        ws = k3g.workspace(k3g.OP_MOE_LAYER, sh)

        def measure(piped):
            cache = k3g.ExpertCache(host, E, arena)

            def step(r):
                k3g.k3g_moe_route(idx, wts, xs[r % n_rot], Wd, bd, K, ws_r)
                if piped:
                    cache.decode_step(y[0], xs[r % n_rot][0], idx.cpu().numpy()[0], wts[0], k3g.EXACT, ws,
                                      copy_stream)
                else:
                    cache.prepare(idx_slot, idx.cpu().numpy(), copy_stream)
                    k3g.k3g_moe_layer(y, xs[r % n_rot], idx_slot, wts, arena, k3g.EXACT, ws)

            for r in range(8):
                step(r)
            torch.cuda.synchronize()
            s0, _, _ = cache.query()
            t0 = time.perf_counter()
            for r in range(steps):
                step(8 + r)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            s1, _, _ = cache.query()
            cache.close()
            copied = s1["bytes_copied"] - s0["bytes_copied"]
            hits, misses = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
            return dt, copied, hits, misses

        dt, copied, hits, misses = measure(False)
        dtp, copied_p, _, _ = measure(True)
        runs.append({"slots": n_slots, "arena_GB": round(n_slots * stride / 1e9, 2), "router_bias_range": bias_range,
                     "steps": steps,
                     "ms_per_step": round(1e3 * dt / steps, 3), "tokens_per_s": round(steps / dt, 1),
                     "hit_rate": round(hits / max(1, hits + misses), 4),
                     "copy_GBps": round(copied / dt / 1e9, 2),
                     "piped_ms_per_step": round(1e3 * dtp / steps, 3), "piped_tokens_per_s": round(steps / dtp, 1),
                     "piped_copy_GBps": round(copied_p / dtp / 1e9, 2)})
        del arena_t, ws
        torch.cuda.empty_cache()
    out["runs"] = runs
    del host
    return out


def copy_calibration(torch, gib):
    """A plain device copy of a known size: each of 5 launches reads and writes n bytes."""
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / 5
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5,
                      "copy_GBps_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)


def host_facts():
    """The host the oracle runs on: CPU model, logical CPUs, OpenMP threads."""
    import oracle

    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "omp_threads": oracle.threads()}


def cpu_baseline(args, src, xs_host, W, b, alg_bytes, T, mode, budget=None, max_experts=320, max_tokens=64):
    """The oracle, as it is, on a bounded sample of the same workload: whole
    steps (fp64 route + layer) of one token at a time. The sample is the
    bench's first tokens, as many (up to max_tokens) as use at most
    max_experts distinct experts between them (their bytes drawn beforehand,
    untimed); passes over the sample repeat until the time budget is spent.
    One token a step: GB/s over the step's algorithmic bytes. More tokens: the
    oracle's cost grows linearly with the tokens (each token's pairs are
    computed on their own, and routing is per token), so the sample's tokens/s
    stands for the batch's."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    K = 16
    budget = args.cpu_seconds if budget is None else budget
    xs_flat = np.concatenate(xs_host, 0)
    sample, used = [], set()
    for i in range(min(max_tokens, xs_flat.shape[0])):
        io, _, _ = oracle.route(xs_flat[i:i + 1], W, b, K)
        ids = {int(e) for e in io.ravel()}
        if sample and len(used | ids) > max_experts:
            break
        used |= ids
        sample.append(i)
    with ThreadPoolExecutor(16) as pool:
        experts = dict(zip(sorted(used), pool.map(src, sorted(used))))
    spent, tokens = 0.0, 0
    while spent < budget:
        for i in sample:
            x = xs_flat[i:i + 1]
            t = time.perf_counter()
            io, wo, _ = oracle.route(x, W, b, K)
            oracle.moe_layer(x, io, wo, {int(e): experts[int(e)] for e in io.ravel()}, 896,
                             oracle.EXACT if mode == 0 else oracle.IDOT)
            spent += time.perf_counter() - t
            tokens += 1
    facts = host_facts()
    # the same steps on one thread, for a quarter of the budget (at least one step)
    n_all = oracle.threads()
    oracle.set_threads(1)
    spent1, tokens1 = 0.0, 0
    try:
        while spent1 < budget / 4 or tokens1 == 0:
            i = sample[tokens1 % len(sample)]
            x = xs_flat[i:i + 1]
            t = time.perf_counter()
            io, wo, _ = oracle.route(x, W, b, K)
            oracle.moe_layer(x, io, wo, {int(e): experts[int(e)] for e in io.ravel()}, 896,
                             oracle.EXACT if mode == 0 else oracle.IDOT)
            spent1 += time.perf_counter() - t
            tokens1 += 1
    finally:
        oracle.set_threads(n_all)
    del experts
    what = "EXACT" if mode == 0 else "IDOT"
    desc = (f"{tokens} token steps over the workload's first {len(sample)} tokens ({len(used)} distinct experts), "
            f"one token at a time, each a whole step (fp64 router + top-16 + 16 {what} SiTU-GLU experts + "
            f"combine), {spent:.1f} s")
    one = {"tokens_per_s": round(tokens1 / spent1, 4), "threads": 1, "seconds": round(spent1, 2),
           "token_steps": tokens1}
    if T == 1:
        one["value"] = round(alg_bytes * tokens1 / spent1 / 1e9, 3)
        return {"value": round(alg_bytes * tokens / spent / 1e9, 3), "unit": "GB/s",
                "tokens_per_s": round(tokens / spent, 4), "cores": facts["omp_threads"], **facts,
                "kind": "oracle", "sample": desc, "single_thread": one}
    one["value"] = one["tokens_per_s"]
    return {"value": round(tokens / spent, 4), "unit": "tokens/s", "cores": facts["omp_threads"], **facts,
            "kind": "oracle",
            "sample": desc + f"; of a {T}-token batch: the oracle's work is linear in the tokens, so the "
                             f"sample's rate stands for the batch's", "single_thread": one}


def cpu_expert(args, ctx, src, n_experts=8):
    """The oracle's one expert on one token (EXACT), on n_experts of the same
    experts the GPU line rotates over (drawn beforehand), for a quarter of the
    CPU time budget on all OpenMP threads and then on one thread: GB/s over
    the same algorithmic bytes as expert_b1.expert_glu."""
    import oracle

    synth = ctx["synth"]
    L, I, E = synth.LATENT, synth.INTER, synth.N_EXPERTS
    ids = [(i * E) // 64 for i in range(n_experts)]  # the first of the 64 the GPU rotates over
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(16) as pool:
        experts = list(pool.map(src, ids))
    x = synth.activations(ctx["seed_bank"], 1, L)[0]
    up_b, dn_b = expert_bytes(L, I)
    nbytes = up_b + dn_b + 2 * L * 4
    budget = args.cpu_seconds / 4

    def timed(limit):
        spent, n = 0.0, 0
        while spent < limit or n == 0:
            t = time.perf_counter()
            oracle.expert_glu(x, experts[n % len(experts)], oracle.EXACT)
            spent += time.perf_counter() - t
            n += 1
        return spent, n

    spent, n = timed(budget)
    n_all = oracle.threads()
    oracle.set_threads(1)
    try:
        spent1, n1 = timed(budget / 4)
    finally:
        oracle.set_threads(n_all)
    facts = host_facts()
    return {"value": round(nbytes * n / spent / 1e9, 3), "unit": "GB/s", "cores": facts["omp_threads"], **facts,
            "kind": "oracle", "calls_per_s": round(n / spent, 3),
            "sample": f"{n} calls of the oracle's EXACT expert on one token over {len(experts)} of the rotated "
                      f"experts, {spent:.1f} s",
            "single_thread": {"value": round(nbytes * n1 / spent1 / 1e9, 3), "threads": 1, "calls": n1,
                              "seconds": round(spent1, 2)}}


def cpu_block(args, ctx, src, n_tokens=4):
    """The oracle's whole LatentMoE block (route, down-projection, routed EXACT
    layer, RMSNorm, up-projection, two shared experts) on the block workload's
    first n_tokens tokens (their experts drawn beforehand), repeated for a
    quarter of the CPU time budget on all OpenMP threads: tokens/s. The block's
    work is per token, so the sample's rate stands for the 256-token batch's."""
    import oracle

    synth = ctx["synth"]
    seed, T, bias_range, _ = synth.WORKLOADS["block_256"]
    H, E, K = synth.HIDDEN, synth.N_EXPERTS, synth.TOP_K
    dense = synth.block_dense(seed)
    W, b = synth.router(seed, E, H, bias_range)
    x = synth.activations(seed, T, H)[:n_tokens]
    io, _, _ = oracle.route(x, W, b, K)
    from concurrent.futures import ThreadPoolExecutor

    ids = sorted(set(io.ravel().tolist()) - {-1})
    with ThreadPoolExecutor(16) as pool:
        experts = dict(zip(ids, pool.map(src, ids)))
    spent, n = 0.0, 0
    while spent < args.cpu_seconds / 4 or n == 0:
        t = time.perf_counter()
        oracle.latent_block(x, W, b, dense, experts, E, K, oracle.EXACT)
        spent += time.perf_counter() - t
        n += 1
    facts = host_facts()
    return {"value": round(n * n_tokens / spent, 4), "unit": "tokens/s", "cores": facts["omp_threads"], **facts,
            "kind": "oracle",
            "sample": f"{n} runs of the oracle's block on the workload's first {n_tokens} tokens "
                      f"({len(experts)} distinct experts), {spent:.1f} s; of a {T}-token batch: the block's work "
                      f"is per token, so the sample's rate stands for the batch's"}


if __name__ == "__main__":
    main()
