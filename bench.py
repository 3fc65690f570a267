#!/usr/bin/env python3
"""Benchmark of one gated sparse decode step on one MI355X.

A step is one pass of the decode hot path for one attention layer of a batch:
pooled-key update for blocks completed at this token (only when a block
completes), gate scores, token-budget block selection, and split-KV sparse
decode with its log-sum-exp merge.  Default workload: batch 16, 32 query /
8 KV heads, head_dim 128, context 65536, 128-token blocks, budget 6553 tokens
-> 51 of 512 blocks kept (90% sparsity), keys of 5% of the blocks mean-shifted.

Several layers' caches are rotated so that consecutive steps read different
memory (as the layers of a model do); with inputs resident in HBM, the value
is effective KV bandwidth: bytes of the kept K/V blocks (plus tail, query,
output and ids) per step divided by the measured step time.

Prints one JSON line.  --gpus N with N > 1 exits: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

from block_sparse_attention_28_amd import inputs, pipeline, probe, seer  # noqa: E402
from block_sparse_attention_28_amd.workloads import (DECODE_L32K, DECODE_L64K_S90, DECODE_WORKLOADS,  # noqa: E402
                                                     RAGGED_DECODE, TINY_DECODE)

HBM_PEAK_GBPS = 8000.0
METRIC = "sparse-decode effective KV GB/s (% of HBM peak) + us/step at 90% sparsity"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DECODE_L64K_S90.name, choices=sorted(DECODE_WORKLOADS))
    ap.add_argument("--layers", type=int, default=8, help="distinct KV caches rotated across steps")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle CPU-baseline budget (0 = skip)")
    ap.add_argument("--cpu-sequences", type=int, default=2)
    ap.add_argument("--prefill-steps", type=int, default=9, help="block-sparse prefill timing: gated and given-block call pairs (0 = skip)")
    ap.add_argument("--mode", default="step", choices=("gate_select", "calls", "step"),
                    help="form of the timed step (the others are timed briefly for context)")
    ap.add_argument("--mode-steps", type=int, default=16, help="steps per form in the context timing (0 = skip)")
    ap.add_argument("--graph-steps", type=int, default=16, help="HIP-graph replays timed (0 = skip)")
    ap.add_argument("--dense", type=int, default=1, help="also time the decode with every block kept (context)")
    ap.add_argument("--other", type=int, default=1, help="time the other decode workloads (context)")
    ap.add_argument("--ceilings", type=int, default=1, help="measure the MFMA rate and the gather-read ceiling")
    return ap.parse_args()


class Layer:
    def __init__(self, w, layer, steps_total, device):
        self.cache = inputs.decode_cache(w, device, layer=layer)
        cap = self.cache["k"].shape[2]
        self.nb_max = cap // w.bs
        self.kpool = torch.zeros((w.B, w.Hkv, self.nb_max, w.d), dtype=torch.float32, device=device)


def code_sha256(files):
    """sha256 over the given C/HIP sources with comments and white space removed, so that
    the hash changes with the code the counters were taken on and not with its comments."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        text = open(os.path.join(ROOT, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()


def measured_traffic(workload_name, record="sparse_decode_traffic.json"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter runs, if they
    were taken on the current kernel code and this workload; else None."""
    path = os.path.join(ROOT, "profiles", record)
    try:
        rec = json.load(open(path))
        if code_sha256(rec["sources"]) != rec["code_sha256"] or rec["workload"] != workload_name:
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def decode_bytes(w, seqlens_host):
    """Algorithmic bytes of one sparse decode launch (kept K/V + tail, q, out, block ids)."""
    kv = 0
    for L in seqlens_host:
        nc, tail = L // w.bs, L % w.bs
        kv += w.Hkv * (min(w.k_max, nc) * w.bs + tail) * w.d * 2 * 2
    q_out = 2 * w.B * w.Hq * w.d * 2
    ids = w.B * w.Hkv * (w.k_max * 4 + 4)
    return kv, kv + q_out + ids


def score_bytes(w, seqlens_host):
    """Gate scores the selection reads: one fp32 per complete block and (b, KV head)."""
    return sum(w.Hkv * (L // w.bs) * 4 for L in seqlens_host)


def graph_step_us(plan, layers, steps, w, args):
    """The step in its timed form (gate, select, decode) captured once per layer as a HIP graph,
    then replayed.  Each replay's output is checked against the eager step's."""
    R = len(layers)
    mode = args.mode
    g_q = torch.empty_like(steps[0]["q"])
    g_sl = torch.empty_like(steps[0]["seqlens"])
    graphs = []
    for l in range(R):
        c = layers[l].cache
        g_q.copy_(steps[l]["q"])
        g_sl.copy_(steps[l]["seqlens"])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.step(g_q, c["k"], c["v"], g_sl, layers[l].kpool, c["wq"], c["wk"], mode=mode)
        graphs.append(g)
    # replay vs eager on the first steps
    for s in range(min(R, 4)):
        lay = layers[steps[s]["layer"]]
        c = lay.cache
        plan.step(steps[s]["q"], c["k"], c["v"], steps[s]["seqlens"], lay.kpool, c["wq"], c["wk"], mode=mode)
        torch.cuda.synchronize()
        ref = plan.out.clone()
        g_q.copy_(steps[s]["q"])
        g_sl.copy_(steps[s]["seqlens"])
        graphs[steps[s]["layer"]].replay()
        torch.cuda.synchronize()
        assert torch.equal(ref, plan.out), "graph replay differs from the eager step"
    n = args.graph_steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(n):
        graphs[s % R].replay()
    e1.record()
    torch.cuda.synchronize()
    one = round(e0.elapsed_time(e1) * 1e3 / n, 2)
    # Four layers' steps in one graph: each replay's own launch cost is shared by four steps.
    G = min(4, R)
    qs = [torch.empty_like(g_q) for _ in range(G)]
    for l in range(G):
        qs[l].copy_(steps[l]["q"])
    g_sl.copy_(steps[0]["seqlens"])
    torch.cuda.synchronize()
    g4 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g4):
        for l in range(G):
            c = layers[l].cache
            plan.step(qs[l], c["k"], c["v"], g_sl, layers[l].kpool, c["wq"], c["wk"], mode=mode)
    c = layers[G - 1].cache
    plan.step(qs[G - 1], c["k"], c["v"], g_sl, layers[G - 1].kpool, c["wq"], c["wk"], mode=mode)
    torch.cuda.synchronize()
    ref = plan.out.clone()
    g4.replay()
    torch.cuda.synchronize()
    assert torch.equal(ref, plan.out), "multi-step graph replay differs from the eager step"
    reps = max(1, n // G)
    e0.record()
    for _ in range(reps):
        g4.replay()
    e1.record()
    torch.cuda.synchronize()
    return {"one_step_per_graph": one, "four_steps_per_graph": round(e0.elapsed_time(e1) * 1e3 / (reps * G), 2)}


def dense_decode_us(w, lay, base_L, dev):
    """Context line: the same decode with every complete block kept (budget = context)."""
    nb_max = lay.nb_max
    L = int(base_L.max())
    shape = pipeline.DecodeShape(w.B, w.Hq, w.Hkv, w.d, w.bs, L, nb_max, w.gate_dim)
    dp = pipeline.DecodePlan(shape, dev)
    sl = base_L.to(torch.int32).to(dev)
    q = inputs.decode_query(w, 0, dev)
    dp.gate_select(q, lay.cache["wq"], lay.cache["wk"], lay.kpool, sl)
    for _ in range(2):
        dp.decode(q, lay.cache["k"], lay.cache["v"], sl)
    torch.cuda.synchronize()
    n = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        dp.decode(q, lay.cache["k"], lay.cache["v"], sl)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    kv = sum(w.Hkv * int(x) * w.d * 2 * 2 for x in base_L.tolist())
    return {"us": round(us, 1), "kept_blocks": int(base_L.min()) // w.bs,
            "effective_GBps": round(kv / (us * 1e-6) / 1e9, 1)}


def ground_truth_context(w, lay, step, plan, dev):
    """Block-level ground truth of the first step's attention (seer_decode_block_mass), its time,
    and how much of the true attention mass the gate's selection captures."""
    c = lay.cache
    nb_max = lay.nb_max
    mass = torch.empty((w.B, w.Hkv, nb_max + 1), dtype=torch.float32, device=dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    wsb = seer.seer_decode_block_mass_workspace_size(w.B, w.Hq, w.Hkv, w.d, nb_max, w.bs, 0)
    ws = torch.zeros((wsb + 3) // 4, dtype=torch.float32, device=dev)
    call = seer.seer_decode_block_mass(step["q"], c["k"], c["v"], step["seqlens"], w.bs, plan.softmax_scale, mass,
                                       out, None, ws, bind=True)
    call()
    torch.cuda.synchronize()
    n = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    plan.gate_select(step["q"], c["wq"], c["wk"], lay.kpool, step["seqlens"])
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    tail = mass[:, :, nb_max]
    blocks = mass[:, :, :nb_max]
    idx = plan.block_idx.long().clamp(min=0)
    valid = (plan.block_idx >= 0).to(mass.dtype)
    captured = (torch.gather(blocks, 2, idx) * valid).sum(-1) + tail
    k = plan.n_sel.max().item()
    best = blocks.topk(k, dim=-1).values.sum(-1) + tail
    kbytes = sum(w.Hkv * int(x) * w.d * 2 * 2 for x in step["L"])
    return {"call": "seer_decode_block_mass", "us": round(us, 1),
            "effective_GBps": round(kbytes / (us * 1e-6) / 1e9, 1),
            "gate_mass_recall": round(captured.mean().item(), 4),
            "best_k_mass": round(best.mean().item(), 4),
            "note": "attention mass of the kept blocks + tail under dense attention; gate weights are random"}


def bf16_table_context(w, lay, step, plan, dev, base_L):
    """The gate + select step from a bf16 pooled-key table: its time and its drift from the fp32 contract."""
    c = lay.cache
    nb_max = lay.nb_max
    k16 = torch.zeros((w.B, w.Hkv, nb_max, w.d), dtype=torch.bfloat16, device=dev)
    ub, uj = pipeline.full_pool_lists(base_L, w.bs, dev)
    seer.seer_pool_k_blocks_ex(c["k"], ub, uj, k16, w.bs)
    sc = torch.empty((w.B, w.Hkv, nb_max), device=dev)
    ix = torch.empty((w.B, w.Hkv, w.k_max), dtype=torch.int32, device=dev)
    ns = torch.empty((w.B, w.Hkv), dtype=torch.int32, device=dev)
    res = {}
    for name, kp, out in (("fp32", lay.kpool, (plan.scores, plan.block_idx, plan.n_sel)), ("bf16", k16, (sc, ix, ns))):
        call = seer.seer_gate_select_ex(step["q"], c["wq"], c["wk"], kp, step["seqlens"], w.bs, plan.gate_scale,
                                        w.k_max, None, *out, bind=True)
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            call()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) * 1e3 / 10, 2)
    a, b = plan.block_idx.cpu(), ix.cpu()
    overlap = sum(len(set(a[i, g].tolist()) & set(b[i, g].tolist())) for i in range(w.B) for g in range(w.Hkv))
    overlap /= (w.B * w.Hkv * max(w.k_max, 1))
    fin = torch.isfinite(plan.scores)
    ref = torch.where(fin, plan.scores, torch.zeros_like(sc))
    diff = torch.where(fin, sc - plan.scores, torch.zeros_like(sc))
    drift = (diff.abs().amax(-1) / ref.abs().amax(-1).clamp(min=1e-30)).max().item()
    return {"gate_select_us_fp32": res["fp32"], "gate_select_us_bf16": res["bf16"],
            "selection_overlap": round(overlap, 4), "max_rel_score_drift": round(drift, 4),
            "note": "kept-set overlap and score drift of a bf16 pooled-key table against the fp32 one"}


def per_head_context(w, lay, step, plan, dev):
    """Per-query-head selection on the first step: gate + per-head select, union decode; bytes against shared."""
    c = lay.cache
    nb_max = lay.nb_max
    sc = torch.empty((w.B, w.Hq, nb_max), device=dev)
    ix = torch.empty((w.B, w.Hq, w.k_max), dtype=torch.int32, device=dev)
    ns = torch.empty((w.B, w.Hq), dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    wsb = seer.seer_sparse_decode_heads_workspace_size(w.B, w.Hq, w.Hkv, w.d, w.k_max, nb_max, w.bs, 0)
    ws = torch.zeros((wsb + 3) // 4 + 4, dtype=torch.float32, device=dev)
    gate = seer.seer_gate_select_heads(step["q"], c["wq"], c["wk"], lay.kpool, step["seqlens"], w.bs,
                                       plan.gate_scale, w.budget, sc, ix, ns, bind=True)
    dec = seer.seer_sparse_decode_heads(step["q"], c["k"], c["v"], step["seqlens"], ix, ns, nb_max, w.bs,
                                        plan.softmax_scale, out, lse, ws, bind=True)
    gate()
    dec()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    n = 10
    t_gate = t_dec = 0.0
    for _ in range(n):
        ev[0].record()
        gate()
        ev[1].record()
        dec()
        ev[2].record()
        torch.cuda.synchronize()
        t_gate += ev[0].elapsed_time(ev[1]) * 1e3 / n
        t_dec += ev[1].elapsed_time(ev[2]) * 1e3 / n
    idx = ix.cpu().view(w.B, w.Hkv, w.G * w.k_max)
    union = sum(len(set(idx[b, g].tolist()) - {-1}) for b in range(w.B) for g in range(w.Hkv))
    shared = int(plan.n_sel.sum().item())
    kv = sum(w.Hkv * (L % w.bs) for L in step["L"]) + union * w.bs   # tokens read: union blocks + tails
    kv_bytes = kv * w.d * 2 * 2
    return {"gate_select_heads_us": round(t_gate, 2), "decode_heads_us": round(t_dec, 2),
            "union_blocks_over_shared": round(union / max(shared, 1), 3),
            "decode_effective_GBps": round(kv_bytes / (t_dec * 1e-6) / 1e9, 1),
            "note": "every query head keeps its own blocks; the decode reads each group's union once"}


def time_launches(fn, n, warm=3):
    """Average microseconds of fn(i) over n calls on the current stream (HIP events)."""
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def decode_workload_context(w, dev, mode, layers=3, steps=16):
    """Another decode workload on rotated layers: the step in the timed form, the step as three
    calls, and the seer_sparse_decode launch (split + merge) with its algorithmic bytes."""
    lay = [Layer(w, l, 0, dev) for l in range(layers)]
    base_L = lay[0].cache["seqlens"].cpu().to(torch.int64)
    shape = pipeline.DecodeShape(w.B, w.Hq, w.Hkv, w.d, w.bs, w.budget, lay[0].nb_max, w.gate_dim)
    plan = pipeline.DecodePlan(shape, dev)
    calls, timed = [], []
    for l, ly in enumerate(lay):
        ub, uj = pipeline.full_pool_lists(base_L, w.bs, dev)
        plan.pool(ly.cache["k"], ly.kpool, ub, uj)
        args = (inputs.decode_query(w, l, dev), ly.cache["k"], ly.cache["v"], ly.cache["seqlens"], ly.kpool,
                ly.cache["wq"], ly.cache["wk"])
        calls.append(plan.bind_step(*args, mode="calls"))
        timed.append(plan.bind_step(*args, mode=mode))

    def step(i, form):
        for c in form[i % layers]:
            c()
    us_step = time_launches(lambda i: step(i, timed), steps)
    us_calls = time_launches(lambda i: step(i, calls), steps)
    us_dec = time_launches(lambda i: calls[i % layers][-1](), steps)
    _, alg = decode_bytes(w, base_L.tolist())
    out = {"workload": w.name, "step_form": mode, "us_step": round(us_step, 2), "us_step_calls": round(us_calls, 2),
           "us_decode_launch": round(us_dec, 2), "bytes_per_launch": int(alg), "num_splits": plan.num_splits}
    if alg > 10_000_000:  # the tiny workload is latency-bound: microseconds only
        gbps = alg / (us_dec * 1e-6) / 1e9
        out.update({"achieved_GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)})
    del lay, plan, calls, timed
    torch.cuda.empty_cache()
    return out


def measured_ceilings(w, layers, plan, steps, dev):
    """Context for the two rooflines: the bf16 MFMA rate this part sustains (both MFMA shapes the
    kernels use, register operands only) and the read rate of the headline decode's own access
    pattern (kept K/V blocks of each layer's first step streamed into LDS, no arithmetic)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {}
    for shape, flops_per_wave_iter in ((16, 16 * 16384), (32, 8 * 32768)):
        wg, iters = cus * 8, 2000
        sink = torch.empty(wg * 256, device=dev)
        us = time_launches(lambda i: probe.mfma_bf16(shape, sink, wg, iters), 3, warm=1)
        res[f"mfma_bf16_{shape}x{shape}_tflops"] = round(wg * 4 * iters * flops_per_wave_iter / (us * 1e-6) / 1e12, 1)
    R = len(layers)
    idx = []
    for l in range(R):
        st = steps[l]
        c = layers[st["layer"]].cache
        plan.gate_select(st["q"], c["wq"], c["wk"], layers[st["layer"]].kpool, st["seqlens"])
        idx.append(plan.block_idx.clone())
    sink = torch.empty(w.B * w.Hkv * plan.num_splits, dtype=torch.int32, device=dev)
    kept = min(w.k_max, min(st_L // w.bs for st_L in steps[0]["L"]))

    def gather(i):
        lay = layers[steps[i % R]["layer"]]
        probe.gather_kv(lay.cache["k"], lay.cache["v"], idx[i % R], kept, w.bs, plan.num_splits, sink)
    us = time_launches(gather, 32)
    kv = w.B * w.Hkv * kept * w.bs * w.d * 2 * 2
    res["gather_read"] = {"us": round(us, 2), "GBps": round(kv / (us * 1e-6) / 1e9, 1),
                          "note": "the headline's kept K/V blocks streamed into LDS as the decode loads them"}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench needs a GPU"
    seer.load()
    dev = torch.device("cuda:0")
    w = DECODE_WORKLOADS[args.workload]
    W, K, R = args.warmup, args.steps, max(1, args.layers)
    total = W + K

    # Per-layer caches with room for the context to grow by one token per R steps.
    from dataclasses import replace
    w_run = replace(w, steps_capacity=max(w.steps_capacity, total // R + 1))
    layers = [Layer(w_run, l, total, dev) for l in range(R)]
    base_L = layers[0].cache["seqlens"].cpu().to(torch.int64)
    nb_max = layers[0].nb_max
    shape = pipeline.DecodeShape(w.B, w.Hq, w.Hkv, w.d, w.bs, w.budget, nb_max, w.gate_dim)
    plan = pipeline.DecodePlan(shape, dev, num_splits=args.num_splits)
    # The pooled-key caches built whole (a1 at start-up), timed on every layer after the first.
    pool_us = []
    ub, uj = pipeline.full_pool_lists(base_L, w.bs, dev)
    for li, lay in enumerate(layers):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        plan.pool(lay.cache["k"], lay.kpool, ub, uj)
        e1.record()
        torch.cuda.synchronize()
        if li > 0 or len(layers) == 1:
            pool_us.append(e0.elapsed_time(e1) * 1e3)
    nc_total = int((base_L // w.bs).sum())
    pool_bytes = nc_total * w.Hkv * w.d * (w.bs * 2 + 4)  # K rows read, fp32 means written
    pool_build = {"us": round(sorted(pool_us)[len(pool_us) // 2], 1), "bytes": pool_bytes,
                  "effective_GBps": round(pool_bytes / (sorted(pool_us)[len(pool_us) // 2] * 1e-6) / 1e9, 1),
                  "note": "seer_pool_k_blocks over every complete block of the batch (the cache built whole)"}

    # Everything a step needs is staged on the device before timing.
    steps = []
    for s in range(total):
        t, l = s // R, s % R
        L = base_L + t
        done = [(b, int(L[b]) // w.bs - 1) for b in range(w.B) if int(L[b]) % w.bs == 0 and t > 0]
        upd = None
        if done:
            upd = (torch.tensor([d[0] for d in done], dtype=torch.int32, device=dev),
                   torch.tensor([d[1] for d in done], dtype=torch.int32, device=dev))
        steps.append({"layer": l, "seqlens": L.to(torch.int32).to(dev), "L": L.tolist(), "upd": upd,
                      "q": inputs.decode_query(w, s, dev)})
    # Each step's launches with their arguments converted once (host marshalling stays out of the loop).
    for st in steps:
        lay = layers[st["layer"]]
        c = lay.cache
        st["pool"] = seer.seer_pool_k_blocks(c["k"], *st["upd"], lay.kpool, w.bs, bind=True) if st["upd"] else None
        st["calls"] = {m: plan.bind_step(st["q"], c["k"], c["v"], st["seqlens"], lay.kpool, c["wq"], c["wk"], mode=m)
                       for m in ("calls", "gate_select", "step")}
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(total)]
    mode = args.mode

    def run_step(s, mode=mode, events=False):
        st = steps[s]
        if events:
            ev[s][0].record(stream)
        if st["pool"] is not None:
            st["pool"]()
        calls = st["calls"][mode]
        for call in calls[:-1]:
            call()
        if events:
            ev[s][1].record(stream)
        calls[-1]()  # the decode launch (split + merge; with the selection in the step form)
        if events:
            ev[s][2].record(stream)

    # A plain elementwise copy of known size (read 256 MiB, write 256 MiB): the
    # reference point that scales hardware byte counters under a profiler.
    cal_x = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    cal_y = torch.empty_like(cal_x)
    torch.mul(cal_x, 1.0, out=cal_y)
    del cal_x, cal_y

    for s in range(W):
        run_step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(W, total):
        run_step(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # The same steps again with events around each step and its last launch.
    for s in range(W, total):
        run_step(s, events=True)
    torch.cuda.synchronize()

    ms_per_step = elapsed * 1e3 / K
    kv_bytes = [decode_bytes(w, steps[s]["L"]) for s in range(W, total)]
    step_us = sorted(ev[s][0].elapsed_time(ev[s][2]) * 1e3 for s in range(W, total))
    mean_kv = sum(b[0] for b in kv_bytes) / K
    mean_alg = sum(b[1] for b in kv_bytes) / K
    value = mean_kv / (ms_per_step * 1e-3) / 1e9
    dom_us = sum(ev[s][1].elapsed_time(ev[s][2]) * 1e3 for s in range(W, total)) / K
    if mode == "step":
        # the selection runs in the decode kernel: its launch also reads the pair's gate scores
        dom_bytes = mean_alg + score_bytes(w, steps[W]["L"])
        dom_name = "seer_select_sparse_decode (select + split decode kernel, LSE merge kernel)"
        traffic_record = "select_sparse_decode_traffic.json"
    else:
        dom_bytes = mean_alg
        dom_name = "seer_sparse_decode (split kernel + LSE merge kernel)"
        traffic_record = "sparse_decode_traffic.json"
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    # The decode launch of the three-call form (split + merge kernels alone), on the same steps.
    dec_calls = [steps[s]["calls"]["calls"][-1] for s in range(W, total)]
    us_dec_calls = time_launches(lambda i: dec_calls[i % len(dec_calls)](), len(dec_calls))
    kept = min(w.k_max, int(base_L.min()) // w.bs)
    ncb = int(base_L.min()) // w.bs

    # Context: the other step forms on the same layers, and the step replayed as a HIP graph.
    modes_us = {}
    for m in ("calls", "gate_select", "step"):
        if args.mode_steps <= 0:
            break
        n = min(args.mode_steps, total)
        for s in range(min(2, n)):
            run_step(s, m)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(n):
            run_step(s, m)
        e1.record()
        torch.cuda.synchronize()
        modes_us[m] = round(e0.elapsed_time(e1) * 1e3 / n, 2)
    graph_us = graph_step_us(plan, layers, steps, w, args) if args.graph_steps > 0 else None
    dense = dense_decode_us(w, layers[0], base_L, dev) if args.dense else None
    gt = ground_truth_context(w, layers[0], steps[0], plan, dev) if args.dense else None
    b16 = bf16_table_context(w, layers[0], steps[0], plan, dev, base_L) if args.dense else None
    ph = per_head_context(w, layers[0], steps[0], plan, dev) if args.dense else None
    ceil = measured_ceilings(w, layers, plan, steps, dev) if args.ceilings else None

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "context": int(base_L[0]) if w.L else [int(base_L.min()), int(base_L.max())],
                   "block_size": w.bs, "budget_tokens": w.budget, "kept_blocks": kept,
                   "sparsity": round(1.0 - kept / max(ncb, 1), 4), "layers_rotated": R,
                   "num_splits": plan.num_splits, "step_form": mode},
        "step_gpu_us": {"p10": round(step_us[K // 10], 2), "p50": round(step_us[K // 2], 2),
                        "p90": round(step_us[(9 * K) // 10], 2)},
        "step_forms_us": modes_us,
        "graph_step_us": graph_us,
        "roofline": {"kernel": dom_name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(w.name, traffic_record) if mode != "gate_select" else None,
                     "bytes_per_launch": int(dom_bytes), "us_per_launch": round(dom_us, 2)},
        "pooled_key_build": pool_build,
        "dense_decode": dense,
        "ground_truth": gt,
        "bf16_pooled_keys": b16,
        "per_head_selection": ph,
        "ceilings": ceil,
    }
    line["roofline"]["seer_sparse_decode_launch"] = {
        "us": round(us_dec_calls, 2), "bytes": int(mean_alg),
        "frac": round(mean_alg / (us_dec_calls * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "traffic": measured_traffic(w.name, "sparse_decode_traffic.json"),
        "note": "split + merge kernels of the three-call form (no selection inside), same steps"}
    if ceil:
        line["roofline"]["frac_of_gather_read"] = round(achieved / ceil["gather_read"]["GBps"], 4)
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(w, layers[0], base_L, plan, args)
    del layers, steps, plan
    torch.cuda.empty_cache()
    if args.other:
        line["other_workloads"] = [decode_workload_context(ow, dev, mode)
                                   for ow in (DECODE_L32K, RAGGED_DECODE, TINY_DECODE)]
    if args.prefill_steps > 0:
        line["secondary_path"] = bench_prefill(args.prefill_steps, dev, ceil)
    print(json.dumps(line), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(counts, bs, d):
    """Algorithmic flops of block-sparse causal attention: 4*bs*bs*d per kept off-diagonal
    block (QK^T and PV), 4*(bs*(bs+1)/2)*d per diagonal block (its causal half)."""
    kept = int(counts.sum())
    diag = counts.numel()
    return (kept - diag) * 4 * bs * bs * d + diag * 4 * (bs * (bs + 1) // 2) * d


def bench_prefill(steps, dev, ceil=None):
    """Gate + MFMA attention of the 32k-token block-sparse causal prefill (keep 1/10)."""
    from block_sparse_attention_28_amd.workloads import PREFILL_L32K as pw
    x = inputs.prefill_inputs(pw, dev)
    nb = (pw.L + pw.bs - 1) // pw.bs
    kmax = seer.seer_block_sparse_prefill_kmax_row(pw.L, pw.bs, pw.keep_num, pw.keep_den)
    blocks = torch.empty((pw.B, pw.H, nb, kmax), dtype=torch.int32, device=dev)
    counts = torch.empty((pw.B, pw.H, nb), dtype=torch.int32, device=dev)
    wsb = seer.seer_block_sparse_prefill_workspace_size(pw.B, pw.H, pw.L, pw.d, pw.bs, pw.gate_dim)
    ws = torch.empty((wsb + 3) // 4, dtype=torch.float32, device=dev)
    out = torch.empty_like(x["q"])
    lse = torch.empty((pw.B, pw.H, pw.L), dtype=torch.float32, device=dev)
    gs, ss = 1 / math.sqrt(pw.gate_dim), 1 / math.sqrt(pw.d)

    def call(given):
        seer.seer_block_sparse_prefill(x["q"], x["k"], x["v"], pw.bs, x["wq"], x["wk"], gs, pw.keep_num,
                                       pw.keep_den, blocks, counts, ss, out, lse, ws, use_given_blocks=given)

    def timed_pair():
        """Medians of gated and given-block calls, interleaved after a warm-up, so that a
        clock that is still ramping up weighs on both alike."""
        for _ in range(3):
            call(False)
            call(True)
        torch.cuda.synchronize()
        got = {False: [], True: []}
        for _ in range(steps):
            for given in (False, True):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call(given)
                e1.record()
                torch.cuda.synchronize()
                got[given].append(e0.elapsed_time(e1) * 1e3)
        med = lambda v: sorted(v)[len(v) // 2]
        # the gate's share: the median of the differences of adjacent calls
        return med(got[False]), med(got[True]), med([a - b for a, b in zip(got[False], got[True])])

    us_total, us_attn, us_gate = timed_pair()
    # ground truth: dense causal attention plus every (query block, key block) mass
    mass = torch.empty((pw.B, pw.H, nb, nb), dtype=torch.float32, device=dev)
    gt = seer.seer_prefill_block_mass(x["q"], x["k"], x["v"], pw.bs, ss, out, mass, lse, bind=True)
    gt()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gt()
    e1.record()
    torch.cuda.synchronize()
    us_gt = e0.elapsed_time(e1) * 1e3
    causal_blocks = nb * (nb + 1) // 2
    dense_flops = (causal_blocks - nb) * 4 * pw.bs * pw.bs * pw.d + nb * 4 * (pw.bs * (pw.bs + 1) // 2) * pw.d
    del mass
    flops = prefill_flops(counts, pw.bs, pw.d)
    tflops = flops / (us_attn * 1e-6) / 1e12
    return {"workload": pw.name, "steps": steps, "us_per_prefill": round(us_total, 1),
            "us_gate": round(us_gate, 1), "us_attention": round(us_attn, 1),
            "kept_blocks_per_head": int(counts[0, 0].sum()), "algorithmic_gflop": round(flops / 1e9, 1),
            "ground_truth": {"call": "seer_prefill_block_mass", "us": round(us_gt, 1),
                             "dense_attention_gflop": round(pw.B * pw.H * dense_flops / 1e9, 1),
                             "note": "dense causal attention + a second QK sweep for every block's mean mass"},
            "roofline": {"kernel": "prefill_attention_kernel", "bound": "mfma", "achieved": round(tflops, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "frac_of_measured_32x32x16": (round(tflops / ceil["mfma_bf16_32x32_tflops"], 4)
                                                       if ceil else None),
                         "traffic": measured_traffic(pw.name, "prefill_attention_traffic.json")}}


def cpu_baseline(w, lay, base_L, plan, args):
    """The fp64 oracle's decode step (gate, select, attention) on a sample of sequences, host cores."""
    import numpy as np

    import oracle
    nseq = max(1, min(args.cpu_sequences, w.B))
    bits = inputs.bf16_bits
    L = [int(x) for x in base_L[:nseq]]
    rows = max(L)
    k = bits(lay.cache["k"][:nseq, :, :rows])
    v = bits(lay.cache["v"][:nseq, :, :rows])
    seq = np.array(L, dtype=np.int32)
    nb = rows // w.bs + 1
    kp = oracle.pool_cache(k, seq, w.bs, nb)   # built once, outside the timing
    wq, wk = bits(lay.cache["wq"]), bits(lay.cache["wk"])
    done, kv, t0 = 0, 0.0, time.perf_counter()
    while True:
        q = bits(inputs.decode_query(w, 10_000 + done, "cuda:0")[:nseq])
        oracle.decode_step(q, k, v, seq, w.bs, w.budget, wq, wk, plan.gate_scale, kp, plan.softmax_scale)
        kv += sum(w.Hkv * (min(w.k_max, x // w.bs) * w.bs + x % w.bs) * w.d * 4 for x in L)
        done += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    el = time.perf_counter() - t0
    cpu_name = platform.processor() or platform.machine()
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_name = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(kv / el / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{nseq} of {w.B} sequences (all {w.Hkv} KV heads), {done} decode steps in {el:.1f} s; "
                      f"pooled cache built once outside the timing",
            "us_per_step_equiv": round(el / done * 1e6 * w.B / nseq, 1), "cpu": cpu_name}


if __name__ == "__main__":
    main()
