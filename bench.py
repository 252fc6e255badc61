#!/usr/bin/env python3
"""Benchmark: DARTree draft-tree construction rounds on one MI355X.

A step is one whole round (head inputs, top-K candidates, depth-by-depth
expansion, global top-B, emission and mask) over one synthetic round of the
qwen3_4b workload (V=151936, L=16, K=64, W=12, B=64, r=256, D=2560, one
request). Rounds run one after another, each on a distinct device-resident
round from a ring larger than the 256 MB Infinity Cache, as in decoding where
each round depends on the previous verification.

Prints one JSON line (see the end of main()).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft-tree builds/sec and us/round at V=151936,L=16,K=64,W=12,B=64 (1 GPU)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--config", default="qwen3_4b")
    ap.add_argument("--ring", type=int, default=128, help="distinct device-resident rounds")
    ap.add_argument("--graph-rounds", type=int, default=16, help="rounds captured per HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-scan-stress", action="store_true",
                    help="skip the logits scan measured at the 64-request shape (311 MB of logits a round)")
    ap.add_argument("--no-serial", action="store_true",
                    help="skip timing the heap-serial construction against the deferred tree kernel")
    ap.add_argument("--no-sizes", action="store_true",
                    help="skip the per-request width/budget timing (four requests of the config)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="if > 0: run only this many eager rounds (for rocprofv3) and exit")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the metric config's timed rounds, rooflines and the CPU baseline")
    ap.add_argument("--no-lmhead", action="store_true", help="skip the fused LM head + top-K timing")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="if > 0: one plain device copy of this many MiB first (calibrates rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE against a known byte count)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              f"(requests would shard across GPUs with no exchange between them)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from diffusion_drafter_tree_amd import inputs as I
    from diffusion_drafter_tree_amd import ops

    torch.cuda.set_device(0)
    cfg = I.CONFIGS[args.config]
    t0 = time.time()
    head = I.make_head(cfg, 0)
    dhead = ops.DeviceHead(head)
    R = max(1, args.ring)
    logits, hin = [], []
    for t in range(R):
        rnd = I.make_round(cfg, 0, t)
        logits.append(ops.to_device(rnd.logits))
        hin.append(ops.to_device(rnd.H if cfg.D > 0 else rnd.h))
    torch.cuda.synchronize()
    print(f"[bench] inputs ready: {R} rounds ({R * logits[0].numel() * logits[0].element_size() / 1e6:.0f} MB of "
          f"logits) in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    if args.copy_mb > 0:
        src = torch.ones(args.copy_mb << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {args.copy_mb} MiB read, {args.copy_mb} MiB written", file=sys.stderr,
              flush=True)
        del src, dst
    rb = ops.RoundBuffers(cfg)
    dims = rb.dims
    stream = torch.cuda.current_stream()

    if args.profile_steps > 0:
        for t in range(args.profile_steps):
            ops.build_round(dims, dhead, logits[t % R], hin[t % R], rb)
        torch.cuda.synchronize()
        print(f"[bench] profiled {args.profile_steps} eager rounds", file=sys.stderr, flush=True)
        return

    # ---- warmup (eager) ------------------------------------------------------
    for t in range(args.warmup):
        ops.build_round(dims, dhead, logits[t % R], hin[t % R], rb)
    torch.cuda.synchronize()

    # ---- graphs of G consecutive ring rounds ---------------------------------
    G = max(1, min(args.graph_rounds, R))
    graphs = []
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(stream)
    with torch.cuda.stream(s_cap):
        for start in range(0, R, G):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s_cap):
                for t in range(start, min(R, start + G)):
                    ops.build_round(dims, dhead, logits[t], hin[t], rb)
            graphs.append((g, min(R, start + G) - start))
    stream.wait_stream(s_cap)
    torch.cuda.synchronize()
    # replay each graph once more as warmup
    for g, _ in graphs:
        g.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly K rounds ----------------------------------------
    K = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done, gi = 0, 0
    plan = []
    while done < K:
        g, n = graphs[gi % len(graphs)]
        if done + n <= K:
            plan.append(("g", g, n))
            done += n
        else:
            plan.append(("e", (gi * G) % R, K - done))
            done = K
        gi += 1
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    ev0.record(stream)
    for kind, obj, n in plan:
        if kind == "g":
            obj.replay()
        else:
            for t in range(n):
                ops.build_round(dims, dhead, logits[(obj + t) % R], hin[(obj + t) % R], rb)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    ms = ev0.elapsed_time(ev1)
    us_round = ms * 1000.0 / K
    builds_per_s = K / (ms / 1000.0)

    # ---- eager rate (host launches, no graph), for reference -------------------
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ne = min(K, 256)
    e0.record(stream)
    for t in range(ne):
        ops.build_round(dims, dhead, logits[t % R], hin[t % R], rb)
    e1.record(stream)
    torch.cuda.synchronize()
    us_eager = e0.elapsed_time(e1) * 1000.0 / ne

    # ---- per-stage kernel durations, live, with HIP events on the launch stream --
    # The library records four events around the launches of each round
    # (scan with head tiles | candidate merge, when separate | tree kernel); eager rounds.
    # Events are created with hipEventDisableSystemFence (timing only: no
    # system-scope cache writeback and invalidation when they complete, which
    # would otherwise sit between the kernels they bracket).
    nk = min(K, 256)
    hev = StageEvents(nk * 4)
    torch.cuda.synchronize()
    for t in range(nk):
        hev.set(t)
        ops.build_round(dims, dhead, logits[t % R], hin[t % R], rb)
    ops.set_stage_events(None)
    torch.cuda.synchronize()
    info = ops.round_plan(dims)
    # event intervals: scan (0-1), separate merge (1-2, when the plan has one), tree (2-3)
    stages = [("scan_kernel", 0)] + ([("merge_kernel", 1)] if info["merge_separate"] else []) + [("tree_kernel", 2)]
    stage_names = [n for n, _ in stages]
    per = {n: [] for n in stage_names}
    tot = []
    skip = min(4, nk // 2)   # the first rounds of the timed pass, when there are enough
    for t in range(skip, nk):
        for n, i in stages:
            per[n].append(hev.elapsed_us(t, i, i + 1))
        tot.append(hev.elapsed_us(t, 0, 3))
    hev.close()
    event_kind = hev.kind
    kern_us = {n: float(np.mean(v)) for n, v in per.items()}

    # algorithmic bytes / flops per launch (the minimal traffic of each stage)
    n, L, V, Kc, W, B, r, D = cfg.n_req, cfg.L, cfg.V, cfg.K, cfg.W, cfg.B, cfg.r, cfg.D
    lsz = 2 if cfg.logits_dtype == "bf16" else 4
    wsz = 2 if cfg.weight_dtype == "bf16" else 4
    rows = n * L
    # slices per row of the logits scan, each leaving a sorted list of K keys (8 B each)
    S_sl = info["scan_slices"]
    lists_bytes = rows * S_sl * Kc * 8 if S_sl > 1 else 0
    cand_bytes = rows * Kc * 8   # candidate ids + logits, written once, read by the tree kernel
    # the scan launch stages A (bf16 in) as fp16 MFMA fragments (out) for the block-decoding kernel
    a_stage = 2 * r * r * 2 if (info["tree_kernel"] and cfg.weight_dtype == "bf16" and r == 256) else 0
    alg = {
        # a1 logits scan + a0 head projection (H, P read once; h written)
        "scan_kernel": {"bytes": rows * V * lsz + (rows * D * wsz + r * D * wsz + rows * r * 4 if D > 0 else 0)
                        + (lists_bytes if S_sl > 1 else cand_bytes) + a_stage,
                        "flops": 2 * rows * D * r},
        "merge_kernel": {"bytes": lists_bytes + cand_bytes, "flops": 0},
        # a2..a5: U rows of every candidate, E rows of the kept nodes, A, h, candidates (or the
        # slice lists it merges), the supertree levels and the outputs
        "tree_kernel": {"bytes": rows * Kc * r * wsz + n * (L - 1) * W * r * wsz + r * r * wsz + rows * r * 4
                        + (lists_bytes + cand_bytes if S_sl > 1 and not info["merge_separate"] else cand_bytes)
                        + n * L * W * 16 + n * B * (20 + ((B + 63) // 64) * 8),
                        "flops": 2 * n * L * W * Kc * r + 2 * n * (L - 1) * W * r * r},
    }
    HBM_PEAK = 8000.0   # GB/s, MI355X HBM3E
    read_peak = measure_read_peak()
    kernels = {}
    for k in stage_names:
        us = kern_us[k]
        gbs = alg[k]["bytes"] / (us * 1e-6) / 1e9 if us > 0 else 0.0
        kernels[k] = {"us": round(us, 3), "alg_bytes": alg[k]["bytes"], "GB_s": round(gbs, 2),
                      "hbm_frac": round(gbs / HBM_PEAK, 5), "alg_flops": alg[k]["flops"]}
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    traffic = measured_traffic(cfg.name)
    cu_read = measure_cu_read_peak()
    roofline = tree_issue_roofline(cfg, kernels, traffic, cu_read) if dom == "tree_kernel" else None
    if roofline is None:
        dk = kernels[dom]
        roofline = {"kernel": dom, "bound": "hbm", "achieved": dk["GB_s"], "peak": HBM_PEAK, "unit": "GB/s",
                    "frac": dk["hbm_frac"], "traffic": traffic.get(dom)}
    sk = kernels["scan_kernel"]
    roofline_scan = {"kernel": "scan_kernel", "bound": "hbm", "achieved": sk["GB_s"], "peak": HBM_PEAK,
                     "unit": "GB/s", "frac": sk["hbm_frac"], "traffic": traffic.get("scan_kernel"),
                     "read_peak_GB_s": read_peak["GB_s"],
                     "frac_of_read_peak": round(sk["GB_s"] / read_peak["GB_s"], 5)}
    round_bytes = alg["scan_kernel"]["bytes"] + alg["tree_kernel"]["bytes"]
    ideal_us = round_bytes / (HBM_PEAK * 1e9) * 1e6
    round_stats = {"p50_us": round(float(np.percentile(tot, 50)), 3), "p99_us": round(float(np.percentile(tot, 99)), 3),
                   "ideal_us_at_hbm_peak": round(ideal_us, 3), "alg_bytes": round_bytes,
                   "round_roofline_frac": round(ideal_us / us_round, 5)}

    # ---- the logits scan where bandwidth decides: 64 requests, K = 512 ----------
    scan_stress = None
    head_stress = None
    if not args.no_scan_stress and not args.no_extras:
        scan_stress = scan_at_stress_shape(HBM_PEAK, read_peak["GB_s"])
        head_stress = head_at_stress_shape()
    other_configs = None
    if not args.no_extras and args.config == "qwen3_4b":
        other_configs = {name: other_config_round(name, HBM_PEAK, read_peak["GB_s"])
                         for name in ("fixed_w4_qwen3_8b", "concurrent_c4")}
        # the 64-request round: four distinct rounds (1.2 GB of logits), graphs of two rounds
        other_configs["stress_64req"] = other_config_round("stress_64req", HBM_PEAK, read_peak["GB_s"], steps=16,
                                                           warmup=2, G=2)
    lmhead = None
    if not args.no_extras and not args.no_lmhead:
        lmhead = lmhead_fused_vs_unfused(read_peak["GB_s"], HBM_PEAK)

    # ---- the heap-serial construction on the same inputs -----------------------
    serial = None
    if not args.no_serial and not args.no_extras and cfg.B <= 511:
        serial = serial_vs_deferred(cfg, dims, dhead, logits[0], hin[0], rb, kern_us["tree_kernel"], us_round)
    verify = None
    if not args.no_serial and not args.no_extras:
        verify = verify_step(cfg, dims, rb)
    sizes = None
    markov = None
    if not args.no_sizes and not args.no_extras:
        sizes = request_sizes(cfg)
        markov = markov_head(cfg, head, logits[0], hin[0])

    # ---- CPU oracle baseline on a bounded sample -------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, head, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(builds_per_s, 1),
        "unit": "builds/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms / K, 6),
        "us_per_round": round(us_round, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in; fp16-split MFMA products, f32 accumulate and scores",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: n_req={n} V={V} L={L} K={Kc} W={W} B={B} beta={cfg.beta} r={r} D={D} "
                               f"logits={cfg.logits_dtype} weights={cfg.weight_dtype}",
                   "ring_rounds": R, "launch": f"hipGraph of {G} rounds per replay",
                   "global_batch": n, "parallelism": "single GPU"},
        "roofline": roofline,
        "roofline_scan": roofline_scan,
        "read_peak": read_peak,
        "cu_read_peak": cu_read,
        "roofline_scan_stress": scan_stress,
        "roofline_head_stress": head_stress,
        "serial_heap": serial,
        "verify_step": verify,
        "request_sizes": sizes,
        "markov_head": markov,
        "other_configs": other_configs,
        "lmhead_topk": lmhead,
        "kernels": kernels,
        "stage_timing": event_kind,
        "plan": info,
        "round": round_stats,
        "us_per_round_eager": round(us_eager, 3),
        "host_seconds_timed": round(t_host, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


KERNEL_SOURCES = {
    "tree_kernel": ["diffusion_drafter_tree_amd/csrc/tree_fast.hip", "diffusion_drafter_tree_amd/csrc/common.h",
                    "diffusion_drafter_tree_amd/csrc/kernels.h"],
    "scan_kernel": ["diffusion_drafter_tree_amd/csrc/scan.hip", "diffusion_drafter_tree_amd/csrc/common.h",
                    "diffusion_drafter_tree_amd/csrc/kernels.h"],
}


def measured_traffic(cfg_name):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of this workload, per kernel, only while the kernel's sources still
    hash to the value recorded with the counters (else the kernel is absent)."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"hbm_traffic_{cfg_name}.md")
    out = {}
    if not os.path.exists(path):
        return out
    rec = None
    for line in open(path):
        if line.startswith("traffic-json:"):
            rec = json.loads(line.split(":", 1)[1])
    for k, files in KERNEL_SOURCES.items():
        if not rec or k not in rec:
            continue
        h = hashlib.sha256()
        for f in files:
            h.update(open(os.path.join(root, f), "rb").read())
        if h.hexdigest()[:16] == rec[k]["src_sha256"]:
            out[k] = rec[k]["bytes"]
    return out


def serial_vs_deferred(cfg, dims, dhead, logits, hin, rb, tree_us, round_us, n_timed=32):
    """dartree_build_serial (one head call per popped node, B pops) on the
    candidates and head inputs of one round, against the deferred tree kernel
    that turns the same inputs into the tree (a2..a5)."""
    import torch

    from diffusion_drafter_tree_amd import ops

    ops.build_round(dims, dhead, logits, hin, rb)
    h = rb.h if cfg.D > 0 else hin
    so = ops.SerialOutputs(cfg)
    for _ in range(3):
        ops.build_serial(dims, dhead, rb.cand_ids, rb.cand_logit, h, so)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_timed):
        ops.build_serial(dims, dhead, rb.cand_ids, rb.cand_logit, h, so)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / n_timed
    return {"kernel": "serial_kernel (B pops, one head call each)", "us_per_build": round(us, 2),
            "deferred_tree_kernel_us": round(tree_us, 2), "deferred_round_us": round(round_us, 2),
            "serial_over_deferred_tree": round(us / tree_us, 2),
            "like_for_like": False,
            "comparison_note": "not like for like: the serial builder computes its head products as fp32 row dot "
                               "products on the VALU with one dependent global round trip a pop, while the "
                               "deferred kernel uses MFMA tiles on prefetched fragments; the ratio bounds the "
                               "construction strategy and the kernel craft together",
            "pages_context": "whole draft rounds with real models on an RTX 6000 Ada: 62.7 ms serial vs 28.5 ms "
                             "deferred (2.2x)"}


def request_sizes(cfg, n_timed=64):
    """dartree_build_round on four requests of the config in one batch, every
    request at the config's (W, B) against per-request widths and budgets
    (W, 2W/3, W/3, W/6 and B, 3B/4, B/2, B/4): the serving knob of choosing
    the tree size per request inside one batch."""
    import torch

    from diffusion_drafter_tree_amd import inputs as I
    from diffusion_drafter_tree_amd import ops

    c4 = cfg.with_(n_req=4, name=cfg.name + "_x4")
    dh = ops.DeviceHead(I.make_head(c4, 0))
    rnd = I.make_round(c4, 0, 0)
    logits = ops.to_device(rnd.logits)
    hin = ops.to_device(rnd.H if c4.D > 0 else rnd.h)
    W, B = c4.W, c4.B
    widths = [W, max(1, 2 * W // 3), max(1, W // 3), max(1, W // 6)]
    budgets = [B, max(1, 3 * B // 4), max(1, B // 2), max(1, B // 4)]
    res = {"requests": 4, "widths": widths, "budgets": budgets}
    for label, wb in (("uniform_us", None), ("per_request_us", (widths, budgets))):
        rb = ops.RoundBuffers(c4)
        if wb is not None:
            rb.set_request_sizes(torch.tensor(wb[0], dtype=torch.int32, device="cuda"),
                                 torch.tensor(wb[1], dtype=torch.int32, device="cuda"))
        for _ in range(3):
            ops.build_round(rb.dims, dh, logits, hin, rb)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n_timed):
            ops.build_round(rb.dims, dh, logits, hin, rb)
        e1.record()
        torch.cuda.synchronize()
        res[label] = round(e0.elapsed_time(e1) * 1000.0 / n_timed, 2)
        if wb is not None:
            res["n_sel"] = rb.n_sel.cpu().tolist()
    res["launch"] = "eager build_round calls, one workgroup a request"
    return res


def markov_head(cfg, head, logits, hin, n_timed=128):
    """dartree_build_round with the Markov-head variant (no A: the kernels skip
    the A s_parent contraction) against the same round with the full head."""
    import torch

    from diffusion_drafter_tree_amd import ops

    res = {}
    for label, markov in (("full_head_us", False), ("markov_head_us", True)):
        dh = ops.DeviceHead(head, markov=markov)
        rb = ops.RoundBuffers(cfg)
        for _ in range(3):
            ops.build_round(rb.dims, dh, logits, hin, rb)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n_timed):
            ops.build_round(rb.dims, dh, logits, hin, rb)
        e1.record()
        torch.cuda.synchronize()
        res[label] = round(e0.elapsed_time(e1) * 1000.0 / n_timed, 2)
    res["launch"] = "eager build_round calls on one round"
    return res


def verify_step(cfg, dims, rb, dh=128, n_timed=32):
    """dartree_verify_tree on the round last built into rb: acceptance against
    a random synthetic target and one tree-attention head (dh = 128) over the
    B draft nodes."""
    import numpy as np
    import torch

    from diffusion_drafter_tree_amd import ops

    n, L, B = cfg.n_req, cfg.L, cfg.B
    rng = np.random.default_rng(3)
    target = ops.to_device(rng.integers(0, cfg.V, (n, L)).astype(np.int32))
    Q, K, V = (ops.to_device(rng.standard_normal((n, B, dh)).astype(np.float32)) for _ in range(3))
    acc_len = torch.zeros((n,), dtype=torch.int32, device="cuda")
    acc_nodes = torch.zeros((n, L), dtype=torch.int32, device="cuda")
    out = torch.zeros((n, B, dh), dtype=torch.float32, device="cuda")
    call = lambda: ops.verify_tree(dims, rb.n_sel, rb.tok, rb.depth, rb.parent, rb.mask, target, Q, K, V, acc_len,
                                   acc_nodes, out)
    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_timed):
        call()
    e1.record()
    torch.cuda.synchronize()
    return {"kernel": "verify_kernel (acceptance + one tree-attention head)", "dh": dh,
            "us": round(e0.elapsed_time(e1) * 1000.0 / n_timed, 2)}


def head_at_stress_shape(n_timed=16):
    """a0 alone (dartree_head_states) at the stress_64req shape: h = P^T H for
    1024 rows, D = 4096, r = 512, bf16 inputs (H ~ N(0, 1), P ~ N(0, 1/D)),
    fp32 output, against the dense bf16 MFMA peak."""
    import numpy as np
    import torch

    from diffusion_drafter_tree_amd import inputs as I
    from diffusion_drafter_tree_amd import ops

    cfg = I.CONFIGS["stress_64req"]
    M, D, r = cfg.n_req * cfg.L, cfg.D, cfg.r
    rng = np.random.default_rng(11)
    H = ops.to_device(I.f32_to_bf16_bits(rng.standard_normal((M, D)).astype(np.float32)))
    Pt = ops.to_device(I.f32_to_bf16_bits((rng.standard_normal((r, D)) / np.sqrt(D)).astype(np.float32)))
    h = torch.empty((M, r), dtype=torch.float32, device="cuda")
    dims = ops.make_dims(cfg)
    for _ in range(4):
        ops.head_states(dims, H, Pt, h)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_timed):
        ops.head_states(dims, H, Pt, h)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / n_timed
    # the vendor library's GEMM on the same operands, timed the same way
    # (torch.matmul on bf16 tensors: hipBLASLt; P made contiguous once, outside
    # the timed calls), for context: what this shape allows a tuned GEMM
    Hb, P = H.view(torch.bfloat16), Pt.view(torch.bfloat16).t().contiguous()
    for _ in range(4):
        torch.matmul(Hb, P)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_timed):
        torch.matmul(Hb, P)
    e1.record()
    torch.cuda.synchronize()
    us_lib = e0.elapsed_time(e1) * 1000.0 / n_timed
    flops = 2 * M * D * r
    peak = 2500.0   # TFLOP/s, dense bf16 MFMA
    tf = flops / (us * 1e-6) / 1e12
    return {"kernel": "head tiles of h = P^T H (64 x 64, LDS-staged, v_mfma_f32_16x16x32_bf16)", "bound": "mfma",
            "workload": f"stress_64req head inputs: M={M} D={D} r={r} bf16, fp32 out", "achieved": round(tf, 1),
            "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4), "us": round(us, 2), "alg_flops": flops,
            "vendor_gemm_us": round(us_lib, 2),
            "vendor_gemm_frac": round(flops / (us_lib * 1e-6) / 1e12 / peak, 4),
            "vendor_gemm": "torch.matmul bf16 (hipBLASLt), bf16 output, same operands"}


def scan_at_stress_shape(hbm_peak, read_peak, n_timed=16):
    """a1 alone (dartree_topk_candidates: the scan launch, then the slice-list
    merge) at the stress_64req shape: 1024 rows of V = 151936 bf16 logits,
    K = 512. Two distinct device-resident rounds (622 MB, over twice the
    Infinity Cache) alternate. Each call's scan and merge launches are timed by
    the library's stage events. A device-to-device copy of one round's logits
    is timed beside it as the achievable-bandwidth reference."""
    import numpy as np
    import torch

    from diffusion_drafter_tree_amd import inputs as I
    from diffusion_drafter_tree_amd import ops

    cfg = I.CONFIGS["stress_64req"]
    lg = [ops.to_device(I.make_round(cfg, 0, t).logits) for t in range(2)]
    rb = ops.RoundBuffers(cfg)
    dims = rb.dims
    info = ops.round_plan(dims)
    for t in range(4):
        ops.topk_candidates(dims, lg[t % 2], rb.cand_ids, rb.cand_logit, rb.ws)
    torch.cuda.synchronize()
    hev = StageEvents(n_timed * 4)
    for t in range(n_timed):
        hev.set(t)
        ops.topk_candidates(dims, lg[t % 2], rb.cand_ids, rb.cand_logit, rb.ws)
    ops.set_stage_events(None)
    torch.cuda.synchronize()
    scan_us = float(np.mean([hev.elapsed_us(t, 0, 1) for t in range(n_timed)]))
    merge_us = float(np.mean([hev.elapsed_us(t, 1, 2) for t in range(n_timed)]))
    hev.close()
    # reference: copy of one round's logits (bytes read + bytes written)
    dst = torch.empty_like(lg[0])
    for _ in range(3):
        dst.copy_(lg[1])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for t in range(8):
        dst.copy_(lg[t % 2])
    e1.record()
    torch.cuda.synchronize()
    nbytes = lg[0].numel() * lg[0].element_size()
    copy_us = e0.elapsed_time(e1) * 1000.0 / 8
    rows = cfg.n_req * cfg.L
    S = info["scan_slices"]
    lists = rows * S * cfg.K * 8 if S > 1 else rows * cfg.K * 8
    alg = nbytes + lists   # logits read once, the slice lists written
    gbs = alg / (scan_us * 1e-6) / 1e9
    return {"kernel": "scan_wide_kernel (logits scan, histogram-ordered selection)", "bound": "hbm",
            "workload": f"stress_64req logits: {rows} rows x V={cfg.V} bf16, K={cfg.K}, {S} slices a row",
            "achieved": round(gbs, 1), "peak": hbm_peak, "unit": "GB/s", "frac": round(gbs / hbm_peak, 4),
            "us": round(scan_us, 2), "alg_bytes": alg, "merge_us": round(merge_us, 2),
            "topk_us": round(scan_us + merge_us, 2),
            "read_peak_GB_s": read_peak, "frac_of_read_peak": round(gbs / read_peak, 4),
            "copy_ref_GB_s": round(2 * nbytes / (copy_us * 1e-6) / 1e9, 1),
            "copy_ref_frac": round(2 * nbytes / (copy_us * 1e-6) / 1e9 / hbm_peak, 4)}


def measure_read_peak(gib=2, n_timed=10):
    """The achievable HBM read rate on this GPU: dartree_stream_read over a
    2 GiB buffer (eight times the Infinity Cache), 16-byte loads from 256
    workgroups, timed with torch events around n_timed passes."""
    import torch

    from diffusion_drafter_tree_amd import ops

    buf = torch.ones((gib << 30) // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(3):
        ops.stream_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_timed):
        ops.stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / n_timed
    nbytes = buf.numel() * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    del buf
    return {"GB_s": round(gbs, 1), "frac_of_8TB_s": round(gbs / 8000.0, 4), "bytes": nbytes, "us": round(us, 2),
            "probe": "dartree_stream_read: one read-only pass, 16-byte loads, 256 x 512 threads"}


def measure_cu_read_peak(mib=8, n_timed=10):
    """The rate one CU pulls from the memory system: dartree_cu_read (one
    workgroup of 1024 threads, 16-byte loads) over an 8 MiB buffer, timed
    with torch events around n_timed passes."""
    import torch

    from diffusion_drafter_tree_amd import ops

    buf = torch.ones((mib << 20) // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(3):
        ops.cu_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_timed):
        ops.cu_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / n_timed
    nbytes = buf.numel() * 4
    del buf
    return {"GB_s": round(nbytes / (us * 1e-6) / 1e9, 2), "bytes": nbytes, "us": round(us, 2),
            "probe": "dartree_cu_read: one read-only pass by one workgroup of 1024 threads, 16-byte loads"}


ISSUE_SOURCES = KERNEL_SOURCES


def measured_issue(cfg_name):
    """Per-launch instruction counts of the tree kernel from the committed
    rocprofv3 counter summary of this workload (SQ_INSTS_VALU and friends),
    while the kernel's sources hash to the recorded value."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"issue_counters_{cfg_name}.md")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("issue-json:"):
            rec = json.loads(line.split(":", 1)[1])
    if not rec or "tree_kernel" not in rec:
        return None
    h = hashlib.sha256()
    for f in ISSUE_SOURCES["tree_kernel"]:
        h.update(open(os.path.join(root, f), "rb").read())
    if h.hexdigest()[:16] != rec["tree_kernel"]["src_sha256"]:
        return None
    return rec["tree_kernel"]


def tree_issue_roofline(cfg, kernels, traffic, cu_read=None):
    """The tree kernel against its issue bound. One request's whole round
    (16 dependent depths) runs in one workgroup on one CU, so the CUs a
    launch occupies are n_req; each issues at most one wave64 VALU
    instruction a cycle (four 16-lane SIMDs, four cycles an instruction) at
    2.4 GHz. achieved = the launch's VALU instructions (rocprofv3
    SQ_INSTS_VALU, from the committed counter summary) / its measured time.
    frac_chip relates the same rate to all 256 CUs. pull: the second bound of
    a one-workgroup kernel, the bytes it moves (algorithmic, and counted)
    against the rate one CU reads at (dartree_cu_read)."""
    rec = measured_issue(cfg.name)
    if rec is None:
        return None
    us = kernels["tree_kernel"]["us"]
    cus = cfg.n_req
    peak = 2.4 * cus   # G wave-instructions/s
    ach = rec["valu_per_launch"] / (us * 1e-6) / 1e9
    return {"kernel": "tree_kernel", "bound": "alu", "achieved": round(ach, 4), "peak": peak,
            "unit": "G VALU wave-instructions/s on the launch's CUs", "frac": round(ach / peak, 4),
            "frac_chip": round(ach / (2.4 * 256), 6), "cus": cus,
            "valu_per_launch": rec["valu_per_launch"], "mfma_per_launch": rec.get("mfma_per_launch"),
            "hbm_frac": kernels["tree_kernel"]["hbm_frac"], "traffic": traffic.get("tree_kernel"),
            "model": "issue: one request's dependent depths run on one CU; peak = one VALU wave64 instruction "
                     "a cycle per CU at 2.4 GHz",
            "pull": tree_pull_bound(cfg, kernels, traffic, cu_read)}


def tree_pull_bound(cfg, kernels, traffic, cu_read):
    """Bytes a launch moves per microsecond against what its CUs can pull
    (one CU a request, each at the measured dartree_cu_read rate)."""
    if not cu_read:
        return None
    us = kernels["tree_kernel"]["us"]
    peak = cu_read["GB_s"] * cfg.n_req
    alg = kernels["tree_kernel"]["alg_bytes"] / (us * 1e-6) / 1e9
    out = {"cu_read_GB_s": cu_read["GB_s"], "cus": cfg.n_req, "peak_GB_s": round(peak, 2),
           "alg_GB_s": round(alg, 2), "alg_frac": round(alg / peak, 4)}
    t = traffic.get("tree_kernel")
    if t:
        tb = t["read"] + t["written"] if isinstance(t, dict) else t
        out["traffic_GB_s"] = round(tb / (us * 1e-6) / 1e9, 2)
        out["traffic_frac"] = round(out["traffic_GB_s"] / peak, 4)
    return out


def other_config_round(name, hbm_peak, read_peak, steps=256, warmup=16, G=16):
    """One more of the five workloads timed like the metric config: a ring of
    distinct device-resident rounds, hipGraph replays of G rounds, the stages
    from the library's events."""
    import numpy as np
    import torch

    from diffusion_drafter_tree_amd import inputs as I
    from diffusion_drafter_tree_amd import ops

    cfg = I.CONFIGS[name]
    # distinct rounds totalling over 600 MB of logits (more than twice the Infinity Cache)
    round_bytes = cfg.n_req * cfg.L * cfg.V * 2
    ring = max(G, -(-600_000_000 // round_bytes) // G * G + G)
    plan = ops.round_plan(ops.make_dims(cfg))
    dh = ops.DeviceHead(I.make_head(cfg, 0))
    lg, hin = [], []
    for t in range(ring):
        r = I.make_round(cfg, 0, t)
        lg.append(ops.to_device(r.logits))
        hin.append(ops.to_device(r.H))
    rb = ops.RoundBuffers(cfg)
    dims = rb.dims
    for t in range(warmup):
        ops.build_round(dims, dh, lg[t % ring], hin[t % ring], rb)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graphs = []
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(stream)
    with torch.cuda.stream(s_cap):
        for start in range(0, ring, G):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s_cap):
                for t in range(start, min(ring, start + G)):
                    ops.build_round(dims, dh, lg[t], hin[t], rb)
            graphs.append(g)
    stream.wait_stream(s_cap)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // G)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    n_rounds = reps * G
    us = e0.elapsed_time(e1) * 1000.0 / n_rounds
    hev = StageEvents(64 * 4)
    for t in range(64):
        hev.set(t)
        ops.build_round(dims, dh, lg[t % ring], hin[t % ring], rb)
    ops.set_stage_events(None)
    torch.cuda.synchronize()
    scan_us = float(np.mean([hev.elapsed_us(t, 0, 1) for t in range(4, 64)]))
    merge_us = float(np.mean([hev.elapsed_us(t, 1, 2) for t in range(4, 64)]))
    tree_us = float(np.mean([hev.elapsed_us(t, 2, 3) for t in range(4, 64)]))
    hev.close()
    rows = cfg.n_req * cfg.L
    scan_bytes = rows * cfg.V * 2
    gbs = scan_bytes / (scan_us * 1e-6) / 1e9
    return {"workload": f"{name}: n_req={cfg.n_req} V={cfg.V} L={cfg.L} K={cfg.K} W={cfg.W} B={cfg.B} "
                        f"beta={cfg.beta} r={cfg.r} D={cfg.D} bf16",
            "us_per_round": round(us, 3), "builds_per_s": round(1e6 / us, 1),
            "request_trees_per_s": round(cfg.n_req * 1e6 / us, 1), "rounds_timed": n_rounds, "ring_rounds": ring,
            "launch": f"hipGraph of {G} rounds per replay",
            "scan_us": round(scan_us, 3), "scan_logits_GB_s": round(gbs, 1),
            "scan_frac_of_8TB_s": round(gbs / hbm_peak, 4), "scan_frac_of_read_peak": round(gbs / read_peak, 4),
            "merge_us": round(merge_us, 3), "tree_kernel_us": round(tree_us, 3),
            "tree_workgroups_per_request": plan["tree_parts"], "stage_timing": "eager rounds, library stage events"}


def lmhead_fused_vs_unfused(read_peak, hbm_peak, n_timed=20):
    """The drafter's LM head fused with the top-K (dartree_lmhead_topk: the
    logits never written) against the unfused pair, a hipBLASLt bf16 GEMM
    writing the logits (torch.matmul) and then the logits scan
    (dartree_topk_candidates), at the metric config's shape: 16 hidden states
    of D = 2560 against a V = 151936 head (778 MB, bf16)."""
    import torch

    from diffusion_drafter_tree_amd import inputs as I
    from diffusion_drafter_tree_amd import ops

    cfg = I.CONFIGS["qwen3_4b"]
    W = I.make_lmhead(cfg, 0)
    X = I.make_lmhead_states(cfg, W, 0, 0)
    rows, D, V, K = cfg.n_req * cfg.L, cfg.D, cfg.V, cfg.K
    dims = ops.make_dims(cfg)
    Wd, Xd = ops.to_device(W), ops.to_device(X)
    del W
    ids = torch.zeros((rows, K), dtype=torch.int32, device="cuda")
    vals = torch.zeros((rows, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.lmhead_workspace_size(dims), dtype=torch.uint8, device="cuda")
    lg = torch.empty((rows, V), dtype=torch.bfloat16, device="cuda")
    wst = torch.empty(ops.workspace_size(dims), dtype=torch.uint8, device="cuda")
    Wt, Xt = Wd.view(torch.bfloat16), Xd.view(torch.bfloat16).reshape(rows, D)

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n_timed):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / n_timed

    fused = timed(lambda: ops.lmhead_topk(dims, Xd, Wd, ids, vals, ws))
    gemm = timed(lambda: torch.matmul(Xt, Wt.t(), out=lg))
    unfused = timed(lambda: (torch.matmul(Xt, Wt.t(), out=lg),
                             ops.topk_candidates(dims, lg.view(torch.int16), ids, vals, wst)))
    head_bytes = V * D * 2
    gbs = head_bytes / (fused * 1e-6) / 1e9
    del Wd
    return {"workload": f"qwen3_4b shape: {rows} hidden states, D={D}, V={V}, K={K}, bf16 head",
            "fused_us": round(fused, 2), "unfused_us": round(unfused, 2), "unfused_gemm_us": round(gemm, 2),
            "fused_over_unfused": round(unfused / fused, 3),
            "fused_head_GB_s": round(gbs, 1), "fused_frac_of_8TB_s": round(gbs / hbm_peak, 4),
            "fused_frac_of_read_peak": round(gbs / read_peak, 4),
            "unfused": "torch.matmul (hipBLASLt) bf16 logits, then dartree_topk_candidates"}


class StageEvents:
    """Four timing events per round for the library's stage hook: HIP events
    created with hipEventDisableSystemFence through the HIP runtime the process
    already uses (the one torch loaded), else torch's events."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.n = n
        self.hip = None
        self.kind = "torch.cuda.Event"
        try:
            hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            evs = []
            for _ in range(n):
                e = ctypes.c_void_p()
                if hip.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000) != 0:   # hipEventDisableSystemFence
                    raise OSError("hipEventCreateWithFlags failed")
                evs.append(e.value)
            self.hip, self.evs = hip, evs
            self.kind = "hipEvent (DisableSystemFence)"
        except OSError:
            import torch
            self.evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def set(self, t):
        from diffusion_drafter_tree_amd import _lib as C
        from diffusion_drafter_tree_amd import ops
        if self.hip is None:
            ops.set_stage_events(self.evs[4 * t:4 * t + 4])
            return
        arr = (self.ct.c_void_p * 4)(*self.evs[4 * t:4 * t + 4])
        st = C.load().dartree_set_stage_events(arr, 4)
        if st != 0:
            raise RuntimeError("dartree_set_stage_events: %s" % C.last_error())

    def elapsed_us(self, t, i, j):
        if self.hip is None:
            return self.evs[4 * t + i].elapsed_time(self.evs[4 * t + j]) * 1000.0
        ms = self.ct.c_float(0.0)
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.evs[4 * t + i], self.evs[4 * t + j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1000.0

    def close(self):
        if self.hip is not None:
            for e in self.evs:
                self.hip.hipEventDestroy(e)
            self.hip = None
            self.evs = []


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rounds(args):
    """Worker: the oracle on seeded rounds ts of config cfg_name, one BLAS
    thread; returns (rounds done, seconds)."""
    cfg_name, ts = args
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        ctx = None
    from diffusion_drafter_tree_amd import inputs as I
    from oracle import dartree_oracle as O
    cfg = I.CONFIGS[cfg_name]
    head = I.make_head(cfg, 0)
    rounds = [I.make_round(cfg, 0, t) for t in ts]
    t0 = time.perf_counter()
    for r in rounds:
        O.round_all(cfg, head, r)
    return len(rounds), time.perf_counter() - t0


def _oracle_heaps(cfg, head, rnd, res):
    """Context beside the deferred oracle: the oracle's two literal heaps on
    the first request of the last timed round, each timed alone (ms). The
    materialised-supertree heap pops the supertree the round built; the
    serial pop-then-correct heap runs the head at every pop over the full
    K-ary tree. Widening the head's tables to fp64 is done once, untimed."""
    from oracle import dartree_oracle as O
    wd = head.dtype
    A, E, U = O.widen(head.A, wd), O.widen(head.E, wd), O.widen(head.U, wd)
    r0 = res[0]
    t0 = time.perf_counter()
    O.heap_materialized(r0.levels, cfg.B)
    t1 = time.perf_counter()
    O.heap_serial_full(r0.cand_ids, r0.cand_vals, r0.h, A, E, U, cfg.beta, cfg.B)
    t2 = time.perf_counter()
    return {"request": 0, "supertree_heap_ms": round(1e3 * (t1 - t0), 3),
            "serial_full_tree_heap_ms": round(1e3 * (t2 - t1), 3),
            "note": "one request of the last round; the serial heap's cost is the head run at each of its B pops"}


def cpu_baseline(cfg, head, budget_s):
    """The oracle as it stands, on the same workload: on 1 host thread over
    distinct seeded rounds until ~budget_s of CPU time, and on every host
    core the process may use (one worker process a core, one BLAS thread
    each) over 100 distinct rounds (rounds/s = rounds / slowest worker's
    time)."""
    import concurrent.futures as cf
    import multiprocessing as mp

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    from diffusion_drafter_tree_amd import inputs as I
    from oracle import dartree_oracle as O

    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    times = []
    heaps = None
    try:
        el = 0.0
        last = None
        while el < budget_s and len(times) < 1000:
            rnd = I.make_round(cfg, 0, 1000 + len(times))
            t0 = time.perf_counter()
            res = O.round_all(cfg, head, rnd)
            dt = time.perf_counter() - t0
            times.append(dt)
            el += dt
            last = (rnd, res)
        heaps = _oracle_heaps(cfg, head, *last) if last else None
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    done = len(times)
    one = {"value": round(done / el, 3), "unit": "builds/s", "cores": 1, "kind": "oracle",
           "median_ms_per_round": round(1e3 * statistics.median(times), 2),
           "sample": f"{done} distinct seeded rounds of {cfg.name} (t = 1000..{999 + done}), numpy fp64, "
                     f"{el:.1f} s of oracle time on 1 host thread (round generation not timed)",
           "literal_heaps": heaps}
    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        ncores = os.cpu_count() or 1
    ncores = max(1, min(ncores, 16))
    n_rounds = 100
    shares = [list(range(i, n_rounds, ncores)) for i in range(ncores)]
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=ncores, mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_rounds, [(cfg.name, sh) for sh in shares if sh]))
    wall = time.perf_counter() - t0
    slowest = max(s for _, s in res)
    many = {"value": round(n_rounds / slowest, 3), "unit": "builds/s", "cores": ncores, "kind": "oracle",
            "sample": f"{n_rounds} distinct seeded rounds of {cfg.name} (t = 0..{n_rounds - 1}) over {ncores} worker "
                      f"processes, one BLAS thread each; rate = rounds / slowest worker's oracle time "
                      f"({slowest:.1f} s; {wall:.1f} s wall with start-up and round generation)"}
    one["cpu_model"] = many["cpu_model"] = _cpu_model()
    one["all_cores"] = many
    return one


if __name__ == "__main__":
    main()
