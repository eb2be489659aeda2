#!/usr/bin/env python3
"""Decode-step benchmark of the AB-Sparse library on one MI355X.

One step = the whole decode hot path for one layer over one batch:
centroid scoring (INT4 by default), top-K, and split attention over the
selected pages merged in the same launch, on inputs already resident in HBM.
By default a step is one abs_select_decode call (the scores, then the top-K
inside the decode launch); --separate times abs_score_select then
abs_sparse_decode instead.  Both forms are timed; "step_call" names the one
`value` is from.  The centroid build (prefill-time) is timed separately and reported
under "build".

Cold-cache honesty: the 256 MB Infinity Cache would hold a step's selected
pages between repeats, so the layer is replicated R times in HBM (distinct
copies of the K/V pools and of the centroid stores) and step i works on copy
i mod R.  By default R is the smallest count, at least 8, whose copies
together hold twice the Infinity Cache in selected pages (8 at 128K x 4,
64 at 32K x 1), within 64 copies and 64 GiB of K/V, so every copy is evicted
before it comes round again.

Prints ONE JSON line (see the "metric" field).  Options:
    --steps K --warmup W   timed / untimed steps (default 200 / 20)
    --workload cfgN        0..4 (default 3: batch 4, 128K context, budget 4096)
    --replicas R           layer copies cycled through (default: see above)
    --layers N             instead of copies of one layer, N distinct layers
                           of the workload (their own data and block maps),
                           cycled through; each step is one layer
    --no-cpu-baseline      skip timing the CPU oracle
    --context N            override the workload's context length (tokens)
    --batch B              override the workload's batch (sequences)
    --block-map M          "drawn" (the workload's seeded map) or 16, 32, 64
                           for a uniform map (all heads one block size)
    --centroid-format F    int4 (default), int4_sym, int8, int4_tensor, bf16
    --warm-cache           also time R steps on one layer copy (Infinity
                           Cache warm), reported as warm_cache_step_us
    --separate             a step is abs_score_select + abs_sparse_decode
    --naive-per-size       also time the per-block-size variant: the heads of
                           each block size as a layer of their own (cache
                           copied per group before timing), one select and
                           one decode call per group and step
    --calibrate-copy MIB   before the timed region, copy MIB MiB device to
                           device three times (a plain copy kernel of known
                           size, the scale for hardware byte counters)
    --gpus N               must be 1 (the library runs on one GPU)
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

PEAK_HBM_GBS = 8000.0
METRIC = "sparse decode attn queries/s per layer at 32K/128K ctx; achieved HBM GB/s vs peak"

# HBM bytes per launch of the kernel the roofline describes (the fused
# top-K + split decode launch, k_select_decode_ws) from rocprofv3 FETCH_SIZE
# and WRITE_SIZE, each scaled by the same counter's reading for a plain copy
# of known size (see profiles/), keyed by (workload, batch, context, block
# map) and by a hash of the kernel sources they were taken with; any other
# shape or source reports null.
TRAFFIC = {
    ("llama8b-128k-b4-bf16", 4, 131072, "drawn", "4c72ecd15774eaf6"): 72015162,
}
KERNEL_SOURCES = ("decode.hip", "device.hpp", "launch.hpp", "decode_layout.hpp", "topk.hpp")   # kernel + its launch layout


INFINITY_CACHE = 256 << 20


def auto_replicas(w, x) -> int:
    """Layer copies whose selected K/V pages add up to twice the Infinity
    Cache (at least 8, at most 64 copies and 64 GiB of K/V)."""
    sz = 2 if x.dtype == "bf16" else 4
    sel_tokens = sum(min(w.token_budget, int(L)) for L in x.seq_lens) * w.num_kv_heads
    step_bytes = max(1, sel_tokens * w.head_dim * 2 * sz)
    kv_bytes = max(1, x.k_cache.nbytes + x.v_cache.nbytes)
    r = max(8, -(-2 * INFINITY_CACHE // step_bytes))
    return int(max(8, min(r, 64, (64 << 30) // kv_bytes)))


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_abs_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="cfg3")
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", type=int, default=0)
    ap.add_argument("--context", type=int, default=0)
    ap.add_argument("--batch", type=int, default=0)
    ap.add_argument("--block-map", default="drawn", choices=["drawn", "16", "32", "64"])
    ap.add_argument("--warm-cache", action="store_true")
    ap.add_argument("--naive-per-size", action="store_true")
    ap.add_argument("--separate", action="store_true")
    ap.add_argument("--centroid-format", default="int4",
                    choices=["int4", "int4_sym", "int8", "int4_tensor", "bf16"])
    return ap.parse_args()


def algorithmic_bytes(x, budget, cap_tokens, code_bits=4):
    """Bytes the method itself must move per decode step (one layer):
    selected K and V, the centroid codes (code_bits per channel) and
    per-channel (scale, lo), q in, out."""
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    esz = 2 if x.dtype == "bf16" else 4
    sel_tokens = sum(cap_tokens(int(L), int(bs)) for L in x.seq_lens for bs in x.block_size)
    kv = sel_tokens * D * esz * 2
    blocks = sum((int(L) + int(bs) - 1) // int(bs) for L in x.seq_lens for bs in x.block_size)
    codes = blocks * D * code_bits // 8
    params = B * Hkv * D * 4 * 2 if code_bits != 16 else 0
    qo = B * Hq * D * esz * 2
    return {"kv": kv, "codes": codes, "params": params, "q_out": qo,
            "decode": kv + qo, "step": kv + codes + params + qo, "sel_tokens": sel_tokens}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU sharding or collectives).", file=sys.stderr)
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py is a single-process, single-GPU benchmark.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_attention_abs_amd import abs as A
    from block_sparse_attention_abs_amd import workload as W

    cfg = int(args.workload.replace("cfg", ""))
    w = W.PRESETS[cfg]
    if args.context:
        w = w.scaled(context=args.context)
    if args.batch:
        w = w.scaled(batch=args.batch)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    x = W.make_layer(w, block_sizes=None if args.block_map == "drawn" else [int(args.block_map)] * w.num_kv_heads)
    print(f"[bench] generated {w.name} in {time.time() - t0:.1f}s, block sizes {x.block_size.tolist()}",
          file=sys.stderr, flush=True)
    B, Hq, D = x.q.shape
    budget = w.token_budget
    sm = float(np.float32(1.0 / np.sqrt(D)))

    base = A.PagedKV.from_host(Hq, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, x.dtype, dev)
    q = A.upload(x.q, dev, x.dtype)
    R = max(1, args.layers or args.replicas or auto_replicas(w, x))
    layers, qs = [base], [q]
    for r in range(1, R):
        if args.layers:
            xr = W.make_layer(w, r, block_sizes=None if args.block_map == "drawn"
                              else [int(args.block_map)] * w.num_kv_heads)
            layers.append(A.PagedKV.from_host(Hq, xr.k_cache, xr.v_cache, xr.page_table, xr.seq_lens, xr.block_size,
                                              xr.dtype, dev))
            qs.append(A.upload(xr.q, dev, xr.dtype))
            del xr
            print(f"[bench] layer {r + 1}/{R} uploaded ({time.time() - t0:.1f}s)", file=sys.stderr, flush=True)
        else:
            layers.append(A.PagedKV(base.k_cache.clone(), base.v_cache.clone(), base.page_table, base.seq_lens,
                                    base.seq_lens_host, base.block_size, base.block_size_host, base.centroid_off,
                                    Hq, x.dtype))
            qs.append(q)
    if args.layers:
        print(f"[bench] {R} distinct layers generated and uploaded in {time.time() - t0:.1f}s", file=sys.stderr,
              flush=True)
    fmt = args.centroid_format
    code_bits = {"int8": 8, "bf16": 16}.get(fmt, 4)
    cents = [A.Centroids.empty(L, fmt) for L in layers]
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)
    ws_b = A.workspace(max(L.workspace_bytes(budget, A.ABS_OP_BUILD) for L in layers), dev)
    ws_s = A.workspace(max(L.workspace_bytes(budget, A.ABS_OP_SELECT) for L in layers), dev)
    ws_d = A.workspace(max(L.workspace_bytes(budget, A.ABS_OP_DECODE) for L in layers), dev)
    ws_sd = A.workspace(max(L.workspace_bytes(budget, A.ABS_OP_SELECT_DECODE) for L in layers), dev)
    cap = max(L.select_capacity(budget) for L in layers)
    sel = torch.zeros((B, w.num_kv_heads, cap), dtype=torch.int32, device=dev)
    cnt = torch.zeros((B, w.num_kv_heads), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, D), dtype=A.torch_dtype(x.dtype), device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)

    # ---- centroid build (prefill-time pass over the whole cache), each copy
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * R)]
    for r in range(R):
        ev[2 * r].record(stream)
        A.abs_build_centroids(layers[r].kv, layers[r].bmap, cents[r].desc, int(ws_b.data_ptr()), ws_b.numel(), sh)
        ev[2 * r + 1].record(stream)
    torch.cuda.synchronize()
    build_ms = sorted(ev[2 * r].elapsed_time(ev[2 * r + 1]) for r in range(R))
    build_med = build_ms[len(build_ms) // 2]
    k_bytes = int(x.seq_lens.sum()) * w.num_kv_heads * D * (2 if x.dtype == "bf16" else 4)
    build_bytes = k_bytes + A.abs_total_blocks(base.kv, base.bmap) * A.abs_centroid_row_bytes(D, A.CENTROID_FORMATS[fmt])

    def select_call(i, st):
        r = i % R
        L = layers[r]
        A.abs_score_select(L.kv, L.bmap, cents[r].desc, int(qs[r].data_ptr()), budget, int(sel.data_ptr()), cap,
                           int(cnt.data_ptr()), int(ws_s.data_ptr()), ws_s.numel(), st)

    def decode_call(i, st):
        r = i % R
        L = layers[r]
        A.abs_sparse_decode(L.kv, L.bmap, int(qs[r].data_ptr()), int(sel.data_ptr()), cap, int(cnt.data_ptr()),
                            budget, sm, int(out.data_ptr()), int(lse.data_ptr()), int(ws_d.data_ptr()), ws_d.numel(),
                            st)

    def separate_step(i, st):
        select_call(i, st)
        decode_call(i, st)

    def fused_step(i, st):
        r = i % R
        L = layers[r]
        A.abs_select_decode(L.kv, L.bmap, cents[r].desc, int(qs[r].data_ptr()), budget, sm, int(sel.data_ptr()),
                            cap, int(cnt.data_ptr()), int(out.data_ptr()), int(lse.data_ptr()),
                            int(ws_sd.data_ptr()), ws_sd.numel(), st)

    step = separate_step if args.separate else fused_step

    # eager warm-up, then each timed unit is a HIP graph of R back-to-back
    # calls (one per layer copy), so host launch cost stays out of the timing
    for i in range(max(args.warmup, R)):
        step(i, sh)
    step(0, sh)   # the diagnostic below reads layer 0's selection
    torch.cuda.synchronize()
    recall = needle_recall(x, sel.cpu().numpy(), cnt.cpu().numpy())
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def capture(fn, n=R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = int(torch.cuda.current_stream().cuda_stream)
            for i in range(n):
                fn(i, st)
        g.replay()
        torch.cuda.synchronize()
        return g

    # the two halves of abs_select_decode on their own (the page's per-stage
    # split): abs_estimate, and abs_topk_decode -- the top-K + split decode
    # launch the roofline describes -- each layer copy on its own workspace,
    # filled by abs_estimate for that copy
    ws_stage = [A.workspace(ws_sd.numel(), dev) for _ in range(R)]

    def estimate_call(i, st):
        r = i % R
        A.abs_estimate(layers[r].kv, layers[r].bmap, cents[r].desc, int(qs[r].data_ptr()), budget,
                       int(ws_stage[r].data_ptr()), ws_stage[r].numel(), st)

    def topk_decode_call(i, st):
        r = i % R
        A.abs_topk_decode(layers[r].kv, layers[r].bmap, int(qs[r].data_ptr()), budget, sm, int(sel.data_ptr()), cap,
                          int(cnt.data_ptr()), int(out.data_ptr()), int(lse.data_ptr()), int(ws_stage[r].data_ptr()),
                          ws_stage[r].numel(), st)

    for i in range(R):
        estimate_call(i, sh)
    torch.cuda.synchronize()
    g_step, g_sel, g_dec = capture(step), capture(select_call), capture(decode_call)
    g_est, g_td = capture(estimate_call), capture(topk_decode_call)
    g_fused, g_sep = capture(fused_step), capture(separate_step)
    torch.cuda.synchronize()

    def timed(g, reps, tail=None):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream()
        torch.cuda.synchronize()
        e0.record(cur)
        for _ in range(reps):
            g.replay()
        if tail is not None:
            tail.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # ---- timed region: exactly K whole steps (K // R replays + a K % R tail)
    K = max(1, args.steps)
    reps = K // R
    g_tail = capture(step, K % R) if K % R else None
    wall0 = time.perf_counter()
    total_ms = timed(g_step, reps, g_tail)
    wall = time.perf_counter() - wall0
    ms_per_step = total_ms / K
    # spread: each replay of R steps timed on its own
    per_rep = np.array([timed(g_step, 1) / R * 1e3 for _ in range(max(10, min(reps, 50)))])
    # per-stage: the same graphs of one stage only, timed the same way
    sreps = max(1, min(reps, 32))
    sel_us = np.array([timed(g_sel, sreps) / (sreps * R) * 1e3 for _ in range(5)])
    dec_us = np.array([timed(g_dec, sreps) / (sreps * R) * 1e3 for _ in range(5)])
    est_us = np.array([timed(g_est, sreps) / (sreps * R) * 1e3 for _ in range(5)])
    td_us = np.array([timed(g_td, sreps) / (sreps * R) * 1e3 for _ in range(5)])
    # both step forms, timed the same way, alternating
    form_us = {"fused": [], "separate": []}
    for _ in range(5):
        form_us["fused"].append(timed(g_fused, sreps) / (sreps * R) * 1e3)
        form_us["separate"].append(timed(g_sep, sreps) / (sreps * R) * 1e3)
    # warm Infinity Cache, for reference: R steps on the same layer copy
    warm_us = None
    if args.warm_cache:
        g_warm = capture(lambda i, st: step(0, st))
        warm_us = round(float(np.median([timed(g_warm, sreps) / (sreps * R) * 1e3 for _ in range(5)])), 3)
    # keeping the centroids current after one appended token per sequence
    # (abs_update_centroids; the last block of every head is recomputed)
    oor = torch.zeros((B, w.num_kv_heads), dtype=torch.int32, device=dev)

    def update_call(i, st):
        r = i % R
        A.abs_update_centroids(layers[r].kv, layers[r].bmap, cents[r].desc, 1, int(oor.data_ptr()), st)

    g_upd = capture(update_call)
    upd_us = float(np.median([timed(g_upd, sreps) / (sreps * R) * 1e3 for _ in range(5)]))

    naive = None
    if args.naive_per_size and args.layers:
        print("[bench] --naive-per-size uses copies of one layer; ignored with --layers", file=sys.stderr)
    elif args.naive_per_size:
        naive = naive_per_size(A, torch, x, layers, q, budget, sm, fmt, R, capture, timed, sreps)

    ab = algorithmic_bytes(x, budget, lambda L, bs: min(L, max(1, budget // bs) * bs), code_bits)
    dec_avg = float(np.median(dec_us))
    td_avg = float(np.median(td_us))
    plan = base.launch_plan(budget)
    # the dominant kernel of the timed step: the top-K + split decode launch
    # (abs_topk_decode) when the layer is served by it, else the split decode
    fused = bool(plan["fused"]) and not args.separate
    kern_us = td_avg if fused else dec_avg
    achieved = ab["decode"] / (kern_us * 1e-6) / 1e9
    queries_per_s = B / (ms_per_step * 1e-3)

    copy_gbs = measured_copy_gbs(torch, dev)
    gather = gather_ceiling(A, torch, x, layers, fused_step, sel, cnt, sh, capture, timed, sreps, R)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, budget, sm, args.cpu_seconds)

    traffic = TRAFFIC.get((w.name, B, int(w.context), args.block_map, kernel_source_hash())) if fused else None
    rec = {
        "metric": METRIC,
        "value": round(queries_per_s, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V, 4 outlier key channels x10, 16 planted needles per head)",
        "config": {"workload": w.name, "batch": B, "context": int(w.context), "q_heads": Hq,
                   "kv_heads": w.num_kv_heads, "head_dim": D, "token_budget": budget, "page_size": 16,
                   "block_sizes": x.block_size.tolist(), "block_map": args.block_map, "centroid_format": fmt,
                   "kv_replicas": None if args.layers else R, "layers": args.layers or 1},
        "roofline": {"bound": "hbm",
                     "kernel": ("k_select_decode_ws (abs_topk_decode: top-K, split decode and merge in one launch)"
                                if fused else "k_sparse_decode_ws (abs_sparse_decode: split, merge in the same launch)"),
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": ab["decode"], "avg_us": round(kern_us, 3),
                     "measured_copy_gbs": round(copy_gbs, 1),
                     "frac_of_measured_copy": round(achieved / copy_gbs, 4),
                     "gather_ceiling": gather,
                     "frac_of_gather_ceiling": round(achieved / gather["gbs"], 4) if gather else None,
                     "decode_only": {"kernel": "k_sparse_decode_ws (abs_sparse_decode)", "avg_us": round(dec_avg, 3),
                                     "frac": round(ab["decode"] / (dec_avg * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}},
        "cpu_baseline": cpu,
        "step": {"algorithmic_bytes": ab["step"], "hbm_gbs": round(ab["step"] / (ms_per_step * 1e-3) / 1e9, 1),
                 "hbm_frac": round(ab["step"] / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                 "step_call": "abs_score_select + abs_sparse_decode" if args.separate else "abs_select_decode",
                 "select_decode_step_us": round(float(np.median(form_us["fused"])), 3),
                 "separate_calls_step_us": round(float(np.median(form_us["separate"])), 3),
                 "estimate_us": round(float(np.median(est_us)), 3), "topk_decode_us": round(td_avg, 3),
                 "launch_plan": plan,
                 "score_select_us": round(float(np.median(sel_us)), 3), "sparse_decode_us": round(dec_avg, 3),
                 "sparse_decode_us_min_max": [round(float(dec_us.min()), 3), round(float(dec_us.max()), 3)],
                 "step_us_p10_p50_p90": [round(float(np.percentile(per_rep, q)), 3) for q in (10, 50, 90)],
                 "warm_cache_step_us": warm_us,
                 "update_centroids_us": round(upd_us, 3),
                 "build_plus_step_us": round(build_med * 1e3 + ms_per_step * 1e3, 3),
                 "wall_s": round(wall, 4)},
        "build": {"ms": round(build_med, 4), "algorithmic_bytes": build_bytes,
                  "hbm_gbs": round(build_bytes / (build_med * 1e-3) / 1e9, 1)},
        "needle_recall": recall,
    }
    if naive is not None:
        rec["naive_per_size"] = naive
    print(json.dumps(rec), flush=True)


def naive_per_size(A, torch, x, layers, q, budget, sm, fmt, R, capture, timed, sreps):
    """The per-block-size variant: for each block size present, the heads of
    that size become a layer of their own (K/V copied per group and layer
    copy, outside the timing); a step calls abs_score_select and
    abs_sparse_decode once per group."""
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    G = Hq // Hkv
    dev = q.device
    groups = []
    for bs in sorted(set(int(b) for b in x.block_size)):
        heads = [h for h in range(Hkv) if int(x.block_size[h]) == bs]
        hidx = torch.tensor(heads, dtype=torch.long, device=dev)
        qidx = torch.tensor([h * G + g for h in heads for g in range(G)], dtype=torch.long, device=dev)
        bs_np = np.full(len(heads), bs, dtype=np.int32)
        gl = []
        for L in layers:
            t = A.PagedKV(L.k_cache[:, hidx].contiguous(), L.v_cache[:, hidx].contiguous(), L.page_table, L.seq_lens,
                          L.seq_lens_host, L.block_size, L.block_size_host, L.centroid_off, len(heads) * G, x.dtype)
            gl.append(t.with_block_sizes(bs_np))
        cents = [A.build_centroids(g, A.Centroids.empty(g, fmt)) for g in gl]
        qg = q[:, qidx].contiguous()
        cap = gl[0].select_capacity(budget)
        grp = dict(bs=bs, heads=heads, layers=gl, cents=cents, q=qg, cap=cap,
                   sel=torch.zeros((B, len(heads), cap), dtype=torch.int32, device=dev),
                   cnt=torch.zeros((B, len(heads)), dtype=torch.int32, device=dev),
                   out=torch.empty((B, len(heads) * G, D), dtype=A.torch_dtype(x.dtype), device=dev),
                   lse=torch.empty((B, len(heads) * G), dtype=torch.float32, device=dev),
                   ws_s=A.workspace(gl[0].workspace_bytes(budget, A.ABS_OP_SELECT), dev),
                   ws_d=A.workspace(gl[0].workspace_bytes(budget, A.ABS_OP_DECODE), dev))
        groups.append(grp)
    torch.cuda.synchronize()

    def sel_g(i, st):
        for g in groups:
            L, c = g["layers"][i % R], g["cents"][i % R]
            A.abs_score_select(L.kv, L.bmap, c.desc, int(g["q"].data_ptr()), budget, int(g["sel"].data_ptr()),
                               g["cap"], int(g["cnt"].data_ptr()), int(g["ws_s"].data_ptr()), g["ws_s"].numel(), st)

    def dec_g(i, st):
        for g in groups:
            L = g["layers"][i % R]
            A.abs_sparse_decode(L.kv, L.bmap, int(g["q"].data_ptr()), int(g["sel"].data_ptr()), g["cap"],
                                int(g["cnt"].data_ptr()), budget, sm, int(g["out"].data_ptr()),
                                int(g["lse"].data_ptr()), int(g["ws_d"].data_ptr()), g["ws_d"].numel(), st)

    def step_g(i, st):
        sel_g(i, st)
        dec_g(i, st)

    st0 = int(torch.cuda.current_stream().cuda_stream)
    for i in range(R):
        step_g(i, st0)
    torch.cuda.synchronize()
    g_step, g_sel, g_dec = capture(step_g), capture(sel_g), capture(dec_g)

    def us(g):
        return round(float(np.median([timed(g, sreps) / (sreps * R) * 1e3 for _ in range(5)])), 3)

    res = {"step_us": us(g_step), "score_select_us": us(g_sel), "sparse_decode_us": us(g_dec),
           "groups": {str(g["bs"]): len(g["heads"]) for g in groups}}
    del groups
    torch.cuda.empty_cache()
    return res


def selected_tiles(page_table, seq_lens, block_size, tile, sel, cnt, k_base, v_base):
    """Device addresses of the K and V tiles ([16][head_dim] of one page and
    KV head, `tile` bytes) of every selected page, in the decode's order: by
    (sequence, head), then selection position, then page, K before V; also
    the byte offsets and which are K."""
    B, Hkv = cnt.shape
    offs = []
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hkv):
            bs = int(block_size[h])
            for j in sel[b, h, :cnt[b, h]]:
                t0, t1 = int(j) * bs, min((int(j) + 1) * bs, L)
                for pg in range(t0 // 16, (t1 + 15) // 16):
                    o = (int(page_table[b, pg]) * Hkv + h) * tile
                    offs.append((o, True))
                    offs.append((o, False))
    o = np.array([a for a, _ in offs], dtype=np.uint64)
    is_k = np.array([k for _, k in offs], dtype=bool)
    return np.where(is_k, np.uint64(k_base) + o, np.uint64(v_base) + o), o, is_k


def gather_ceiling(A, torch, x, layers, fused_step, sel, cnt, sh, capture, timed, sreps, R):
    """The rate at which the GPU gathers the K/V tiles a decode step selects,
    with none of the decode's arithmetic (abs_gather_tiles, the decode's
    non-temporal loads): for each layer copy its own selection's tiles, one
    launch per copy in a graph as for the kernels, the best over launch
    shapes (workgroups x tiles in flight per wavefront).  Layer 0's words
    are checked against the host arrays (XOR).  None where the tiles are not
    4 KiB (bf16, head_dim 128)."""
    D = x.k_cache.shape[3]
    if x.dtype != "bf16" or D != 128:
        return None
    addrs = []
    for r in range(R):
        fused_step(r, sh)
        torch.cuda.synchronize()
        Lr = layers[r]
        a, o, is_k = selected_tiles(Lr.page_table.cpu().numpy(), Lr.seq_lens_host, Lr.block_size_host, 4096,
                                    sel.cpu().numpy(), cnt.cpu().numpy(), Lr.k_cache.data_ptr(),
                                    Lr.v_cache.data_ptr())
        if r == 0:
            want = 0
            for cache, m in ((x.k_cache, is_k), (x.v_cache, ~is_k)):
                words = cache.reshape(-1).view(np.uint32)
                idx = (o[m] // 4)[:, None] + np.arange(1024, dtype=np.uint64)[None, :]
                want ^= int(np.bitwise_xor.reduce(words[idx].ravel()))
            n0 = len(a)
        addrs.append(torch.from_numpy(a.view(np.int64)).to(sel.device))
    n = len(addrs[0])
    if any(len(t) != n for t in addrs):
        return None
    best, shapes = None, []
    for wgs in (256, 512, 1024, 2048):
        out = torch.zeros((wgs,), dtype=torch.int32, device=sel.device)
        for u in (1, 2, 4, 8):
            def call(i, st, wgs=wgs, u=u, out=out):
                A.abs_gather_tiles(int(addrs[i % R].data_ptr()), n, 4096, wgs, u, int(out.data_ptr()), st)
            call(0, sh)
            torch.cuda.synchronize()
            got = int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)))
            if got != want:
                raise SystemExit(f"gather probe read wrong words (workgroups {wgs}, in flight {u})")
            g = capture(call)
            us = float(np.median([timed(g, sreps) / (sreps * R) * 1e3 for _ in range(5)]))
            gbs = n * 4096 / (us * 1e-6) / 1e9
            shapes.append([wgs, u, round(gbs, 1)])
            if best is None or gbs > best["gbs"]:
                best = {"gbs": round(gbs, 1), "avg_us": round(us, 3), "workgroups": wgs, "in_flight": u,
                        "tiles": n, "bytes": n * 4096, "checked_tiles": n0}
            del g
    best["shapes"] = shapes              # [workgroups, tiles in flight, GB/s] of every launch shape tried
    return best


def measured_copy_gbs(torch, dev, nbytes=1 << 30, reps=5):
    """This GPU's streaming rate as a plain device copy sees it: bytes read
    plus bytes written per second over `reps` copies of 1 GiB (HIP events)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def needle_recall(x, sel, cnt):
    """Diagnostic, not asserted: per block size, the fraction of planted
    needles whose block the GPU selected."""
    hit, tot = {}, {}
    for (b, h), k in np.ndenumerate(cnt):
        bs = int(x.block_size[h])
        chosen = set(sel[b, h, :k].tolist())
        for t in x.needle_pos[b, h]:
            if t < 0:
                continue
            tot[bs] = tot.get(bs, 0) + 1
            hit[bs] = hit.get(bs, 0) + (int(t) // bs in chosen)
    return {str(bs): round(hit[bs] / tot[bs], 4) for bs in sorted(tot)}


def cpu_baseline(x, budget, sm, seconds):
    """The oracle as it stands (oracle/, plain C, fp64, OpenMP over (b, h)) on
    the same host arrays: whole decode steps (score + select + attend over the
    full batch) repeated for about `seconds` on all host threads, with the
    stages timed apart; then one step on a single thread.  Its centroids are
    built once, timed on their own."""
    import oracle as O
    t0 = time.perf_counter()
    c = O.centroids(x.k_cache, x.page_table, x.seq_lens, x.block_size, x.dtype)
    qz = O.quantize(c, x.seq_lens, x.block_size)
    build_s = time.perf_counter() - t0
    cap = O.sel_capacity(x.seq_lens, x.block_size, budget)

    def one_step():
        a = time.perf_counter()
        s = O.scores(x.q, qz, x.seq_lens, x.block_size, x.dtype)
        sel, cnt = O.select(s, x.seq_lens, x.block_size, budget, cap)
        b = time.perf_counter()
        O.attend(x.q, x.k_cache, x.v_cache, x.page_table, x.seq_lens, x.block_size, sel, cnt, sm, x.dtype)
        return b - a, time.perf_counter() - b

    threads = O.max_threads()
    n, t_sel, t_att, t0 = 0, 0.0, 0.0, time.perf_counter()
    while True:
        a, b = one_step()
        t_sel += a
        t_att += b
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    O.set_threads(1)
    try:
        a, b = one_step()
    finally:
        O.set_threads(threads)
    B = x.q.shape[0]
    return {"value": round(n * B / el, 3), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} full decode steps (batch {B}) of the same workload, {el:.1f}s on {threads} threads; "
                      f"centroids built once outside the timing",
            "score_select_ms": round(t_sel / n * 1e3, 3), "attend_ms": round(t_att / n * 1e3, 3),
            "build_ms": round(build_s * 1e3, 1), "single_thread_step_ms": round((a + b) * 1e3, 2)}


if __name__ == "__main__":
    main()
