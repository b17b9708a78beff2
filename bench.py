#!/usr/bin/env python3
"""Decode-step benchmark of query-guided block-sparse attention on one MI355X.

Workload: the GQA 128K decode workload (batch 4, 32 query / 8 KV heads,
head_dim 128, context 131072, bf16 KV with 16 needle blocks per KV head;
Quest min/max summaries over 32-token blocks, top-128 blocks + 512-token
window, selection shared by the 4 query heads of a KV group). Inputs are
seeded synthetic data (synth/), resident in HBM before timing starts.

One step = the whole decode-time path through the C ABI, hs_decode_step in
one launch: refresh of the growing last block's summary, selection (score
all 4096 blocks per unit, top-k, window union) and exact softmax attention
over the selected blocks (--path separate: hs_build_summaries,
hs_select_blocks, hs_sparse_decode as three launches, same results).

The per-step working set (summaries + selected KV, ~143 MB) would fit in the
256 MiB Infinity Cache, so the timed loop rotates over `--copies` identical
copies of the inputs (at 8 copies every reuse is ~1 GB of traffic apart),
which makes each step read from HBM. Steps are HIP-graph replays: one graph
holds a round of 8 steps, one on each copy (unless --no-graph).

With the headline line come: per-step p10 / median / p90, the same box's
streaming ceilings, one-step figures of the 4K, 32K and 256K two-level
workloads and of the 8-layer shared-selection workload, the f1-f4 figures
(decode loop, ratio + reserve set, token stage, block cache) and the CPU
oracle's baseline at 1 and N threads (see --figures, --headline-only,
--no-cpu).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def log(msg):
    print("[bench %s] %s" % (time.strftime("%H:%M:%S"), msg), file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--copies", type=int, default=0,
                    help="input copies the timed loop rotates over; 0: 8 when a step's working "
                         "set fits the 256 MiB Infinity Cache, else 1")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--event-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="seconds of oracle work per CPU-baseline measurement (1 thread, N threads)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--path", choices=["fused", "separate"], default="fused")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the decode loop, ratio, token-stage and block-cache figures (profiling "
                         "runs: their launches would mix into the kernel averages)")
    ap.add_argument("--figures", default="loop,ratio,tokens,cache,shared,configs",
                    help="comma-separated figures to add after the headline (profiling runs pick "
                         "one): loop, ratio, tokens, cache, shared, configs")
    ap.add_argument("--loop-steps", type=int, default=64,
                    help="steps of the timed decode loop (append + step); 0 skips it")
    ap.add_argument("--mode", choices=["step", "copy", "shared"], default="step",
                    help="copy: plain device-to-device copy of known size (counter calibration); "
                         "shared: only the 8-layer shared-selection figure (its kernel trace)")
    return ap.parse_args()


def source_digest(files):
    """sha256 over the given sources (relative to the repository root)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


_CSRC = "hierarchical_sparse_attention_amd/csrc/"
KERNEL_SOURCES = {
    "hs_sparse_decode": [_CSRC + f for f in ("decode.hip", "decode_impl.h", "hs_internal.h")],
    "hs_select_blocks": [_CSRC + f for f in ("select.hip", "select_impl.h", "hs_internal.h")],
    "hs_decode_step": [_CSRC + f for f in ("step.hip", "select_impl.h", "decode_impl.h",
                                           "summ_impl.h", "hs_internal.h")],
    # two levels: the launch before the fused kernel (refreshes + coarse selection)
    "hs_two_level_head": [_CSRC + f for f in ("select.hip", "select_impl.h", "summ_impl.h",
                                              "hs_internal.h")],
    # token level: the selection kernel with token rows, and the token-list attention
    "hs_select_tokens": [_CSRC + f for f in ("select.hip", "select_impl.h", "hs_internal.h")],
    "hs_sparse_decode_tokens": [_CSRC + f for f in ("decode.hip", "decode_impl.h",
                                                    "hs_internal.h")],
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current source of the kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec["hbm_bytes_per_launch"]


def step_bytes(w, ids, cnt):
    """Algorithmic bytes of one decode step of workload w whose selection is
    ids / cnt (host arrays): the summary rows the selection scores (every fine
    block; with two levels every coarse block and the fine blocks inside the
    kept coarse blocks), the refresh of the growing block of each level (its
    tokens' K rows read, its summary row written), the K and V rows of the
    selected tokens, and q, ids and outputs."""
    import numpy as np
    esize = 2 if w.dtype == "bf16" else 4
    lens = w.seq_lens_array()
    tokens = 0
    for b in range(w.batch):
        for g in range(w.hkv):
            sel = ids[b, g, :cnt[b, g]].astype(np.int64)
            tokens += int(np.minimum(w.S, lens[b] - sel * w.S).sum())
    row = w.d * 4 if w.kind == "mean" else 2 * w.d * esize
    q_bytes = w.batch * w.hq * w.d * esize
    id_bytes = int(cnt.sum()) * 4 + w.units * 4
    refresh = w.units * (w.S * w.d * esize + row)
    if w.top_k_coarse:
        crow = w.d * 4  # coarse level: mean-pooled keys
        ratio = w.coarse_S // w.S
        cand = min(w.nb, min(w.top_k_coarse, w.nc) * ratio)
        select = w.units * (w.nc * crow + cand * row) + q_bytes + id_bytes
        refresh += w.units * (w.coarse_S * w.d * esize + crow)
    else:
        select = w.units * w.nb * row + q_bytes + id_bytes
    decode = tokens * w.d * esize * 2 + q_bytes + id_bytes + w.batch * w.hq * w.d * 4
    return {"select": select, "decode": decode, "refresh": refresh,
            "step": select + decode + refresh, "kv_tokens": tokens}


def dominant_traffic(w, nb):
    """Measured HBM bytes of the step's dominant kernel, k_step (from the
    committed counter summary of this workload, when it was taken on the
    current sources), next to that kernel's own algorithmic bytes: with two
    levels the coarse selection and the table refreshes are separate launches,
    so k_step's share is the fine candidates' rows and the attention."""
    hbm = measured_traffic("hs_decode_step", w.name)
    if hbm is None:
        return None
    if w.top_k_coarse:
        esize = 2 if w.dtype == "bf16" else 4
        row = w.d * 4 if w.kind == "mean" else 2 * w.d * esize
        cand = min(w.nb, min(w.top_k_coarse, w.nc) * (w.coarse_S // w.S))
        alg = nb["decode"] + w.units * cand * row
    else:
        alg = nb["step"]
    return {"kernel": "k_step", "hbm_bytes_per_launch": hbm, "algorithmic_bytes": alg,
            "ratio": hbm / alg}


def needle_recall(w, ids, cnt):
    """Fraction of the planted needle blocks (every unit) that the selection kept."""
    if not w.needles:
        return None
    hit = tot = 0
    for b in range(w.batch):
        for g in range(w.hkv):
            nd = set(w.needle_blocks(b, g).tolist())
            hit += len(nd & set(ids[b, g, :cnt[b, g]].tolist()))
            tot += len(nd)
    return hit / tot if tot else None


def auto_copies(w):
    """8 input copies when a step's working set (summaries + the largest
    selection's K/V) fits the 256 MiB Infinity Cache, so that rotating over
    them makes every step read HBM; 1 otherwise."""
    esize = 2 if w.dtype == "bf16" else 4
    row = w.d * 4 if w.kind == "mean" else 2 * w.d * esize
    est = w.units * (w.nb * row + w.max_selected * w.S * w.d * esize * 2)
    return 8 if est < (256 << 20) else 1


def copy_mode(args):
    """Plain device copy of a known size: 1 GiB read + 1 GiB written per call.
    Run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to calibrate the counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "calls": args.steps,
                      "GBps": 2 * n / dt / 1e9}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the path is measured on one GPU's share of the "
              "work (--gpus %d was requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        copy_mode(args)
        return
    if args.mode == "shared":
        import torch
        torch.cuda.set_device(0)
        res = shared_selection_timing(torch.cuda.Stream(), args.event_steps)
        print(json.dumps({"mode": "shared", "figure": "shared_selection", "reps": args.event_steps,
                          "config": {"workload": res["workload"]}, "shared_selection": res}),
              flush=True)
        return
    import numpy as np
    import torch

    import hierarchical_sparse_attention_amd as hs
    from synth import device as sdev
    from synth.workloads import CONFIGS

    w = CONFIGS[args.config]
    assert w.layers == 1, "the 8-layer workload is the shared_selection figure (--mode shared)"
    n_copies = args.copies or auto_copies(w)
    torch.cuda.set_device(0)
    dev = "cuda"
    stream = torch.cuda.Stream()
    esize = 2 if w.dtype == "bf16" else 4

    # ------------------------------------------------------------ inputs
    t = time.time()
    log("generating %s inputs" % w.name)
    kp0, vp0 = sdev.make_pools(w)
    pt = sdev.page_table_tensor(w)
    sl = sdev.seq_lens_tensor(w)
    q0 = sdev.q_tensor(w)
    torch.cuda.synchronize()
    log("inputs on device in %.1f s (%.2f GB of K/V)" % (time.time() - t,
                                                         2 * kp0.numel() * esize / 1e9))
    cap = w.max_selected
    kc = w.top_k_coarse
    copies = []
    for c in range(n_copies):
        kp = kp0 if c == 0 else kp0.clone()
        vp = vp0 if c == 0 else vp0.clone()
        kv = hs.KVCache(kp, vp, pt, sl, w.T)
        fine = hs.Summaries.empty(kv, w.kind, w.S)
        coarse = hs.Summaries.empty(kv, "mean", w.coarse_S) if kc else None
        q = q0 if c == 0 else q0.clone()
        ids = torch.zeros((w.batch, w.hkv, cap), dtype=torch.int32, device=dev)
        cnt = torch.zeros((w.batch, w.hkv), dtype=torch.int32, device=dev)
        out = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device=dev)
        ws_s = hs.workspace(hs.hs_select_workspace_size(kv, fine, w.hq, w.top_k, w.window, cap,
                                                        coarse, kc), dev)
        ws_d = hs.workspace(hs.hs_decode_workspace_size(kv, w.hq, w.S, cap), dev)
        ws_f = hs.workspace(hs.hs_select_decode_workspace_size(kv, fine, w.hq, w.top_k, w.window,
                                                               cap, coarse, kc), dev)
        copies.append(dict(kv=kv, fine=fine, coarse=coarse, q=q, ids=ids, cnt=cnt, out=out,
                           ws_s=ws_s, ws_d=ws_d, ws_f=ws_f))
    torch.cuda.synchronize()

    # full summary build (prefill phase; reported separately, not part of a step)
    build_ms = []
    for c in copies:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        hs.hs_build_summaries(c["kv"], c["fine"], 0, stream=stream)
        e1.record(stream)
        if kc:
            hs.hs_build_summaries(c["kv"], c["coarse"], 0, stream=stream)
        e1.synchronize()
        build_ms.append(e0.elapsed_time(e1))
    torch.cuda.synchronize()
    row = w.d * 4 if w.kind == "mean" else 2 * w.d * esize
    build_bytes = w.units * (w.T * w.d * esize + w.nb * row)
    if kc:  # the coarse table is built from the tokens too
        build_bytes += w.units * (w.T * w.d * esize + w.nc * w.d * 4)
    build_avg = float(np.mean(build_ms[1:] if len(build_ms) > 1 else build_ms))
    log("full summary build: %.3f ms, %.0f GB/s" % (build_avg, build_bytes / build_avg / 1e6))

    last_block = (w.T - 1) // w.S
    names = ["hs_build_summaries(last block)", "hs_select_blocks", "hs_sparse_decode",
             "hs_select_decode", "hs_decode_step"]
    if kc:
        names.append("hs_build_summaries(last coarse block)")
    for c in copies:
        c["calls"] = [
            hs.prepare_build_summaries(c["kv"], c["fine"], last_block, stream),
            hs.prepare_select_blocks(c["kv"], c["q"], c["fine"], w.top_k, w.window, c["ids"],
                                     c["cnt"], c["ws_s"], stream, c["coarse"], kc),
            hs.prepare_sparse_decode(c["kv"], c["q"], w.S, c["ids"], c["cnt"], c["out"],
                                     c["ws_d"], stream),
            hs.prepare_select_decode(c["kv"], c["q"], c["fine"], w.top_k, w.window, c["ids"],
                                     c["cnt"], c["out"], c["ws_f"], stream, c["coarse"], kc),
            hs.prepare_decode_step(c["kv"], c["q"], c["fine"], w.top_k, w.window, last_block,
                                   c["ids"], c["cnt"], c["out"], c["ws_f"], stream, c["coarse"],
                                   kc),
        ]
        if kc:
            c["calls"].append(hs.prepare_build_summaries(c["kv"], c["coarse"],
                                                         last_block * w.S // w.coarse_S, stream))
    step_calls = [4] if args.path == "fused" else ([0, 5, 1, 2] if kc else [0, 1, 2])

    def step(c):
        for j in step_calls:
            c["calls"][j]()

    # ------------------------------------------------ per-call event timing
    # Each entry point is captured as a graph of back-to-back launches, one per
    # input copy, and timed with events on the launch stream: the average per
    # launch is the kernel's duration plus the dispatch gap between graph nodes,
    # comparable with the kernel trace of rocprofv3.
    with torch.cuda.stream(stream):
        for c in copies:  # fill every copy's ids (the decode's input)
            step(c)
    torch.cuda.synchronize()
    call_ms = []
    for j in range(len(names)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in copies:
                c["calls"][j]()
        torch.cuda.synchronize()
        replay_t = replay_ms(g, stream, args.event_steps)
        call_ms.append(float(replay_t.mean()) / len(copies))
        del g
    call_ms = np.array(call_ms)
    log("per-call mean ms: refresh %.4f select %.4f decode %.4f select+decode %.4f step %.4f" %
        tuple(call_ms[:5]))

    # ---------------------------------------------------------- graphs
    # One graph per input copy holds one step; one round graph holds a step on
    # every copy in turn (at least 8 steps: a single copy is stepped 8 times),
    # so that the timed loop pays one graph launch per round of complete
    # steps, as a decode loop that captures its steps would.
    graphs = round_graph = None
    per_round = max(len(copies), 8)
    if not args.no_graph:
        graphs = []
        for c in copies:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(c)
            graphs.append(g)
        round_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(round_graph, stream=stream):
            for i in range(per_round):
                step(copies[i % len(copies)])
        torch.cuda.synchronize()

    def run(i):
        if graphs is not None:
            graphs[i % len(graphs)].replay()
        else:
            step(copies[i % len(copies)])

    def run_steps(n):
        """n steps: whole rounds from the round graph, the rest one by one."""
        i = 0
        if round_graph is not None:
            for _ in range(n // per_round):
                round_graph.replay()
            i = n // per_round * per_round
        for j in range(i, n):
            run(j)

    # ------------------------------------------------------- timed loop
    with torch.cuda.stream(stream):
        run_steps(args.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(args.steps)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # each step's own duration on the GPU, for the median and p10 / p90: an
    # event after every single-step replay (untimed by the loop above)
    n_q = max(args.steps, 20)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_q + 1)]
    with torch.cuda.stream(stream):
        step_ev[0].record(stream)
        for i in range(n_q):
            run(i)
            step_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(n_q)])
    step_q = {"steps": n_q, "p10": float(np.percentile(per_step, 10)),
              "median": float(np.median(per_step)), "p90": float(np.percentile(per_step, 90))}

    # warm (cache-resident) figure: one copy back to back, for context only
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            run(0) if graphs is None else graphs[0].replay()
        torch.cuda.synchronize()
        tw0 = time.perf_counter()
        for i in range(args.steps):
            run(0) if graphs is None else graphs[0].replay()
        torch.cuda.synchronize()
        tw1 = time.perf_counter()
    warm_ms = (tw1 - tw0) * 1e3 / args.steps

    # ----------------------------------------------- algorithmic bytes
    c0 = copies[0]
    ids = c0["ids"].cpu().numpy()
    cnt = c0["cnt"].cpu().numpy()
    nbytes = step_bytes(w, ids, cnt)
    bytes_decode, bytes_select = nbytes["decode"], nbytes["select"]
    bytes_refresh, bytes_step, kv_tokens = nbytes["refresh"], nbytes["step"], nbytes["kv_tokens"]
    log("bytes/step: select %.1f MB, decode %.1f MB (%d KV tokens), refresh %.2f MB" % (
        bytes_select / 1e6, bytes_decode / 1e6, kv_tokens, bytes_refresh / 1e6))
    recall = needle_recall(w, ids, cnt)

    dec_ms = float(call_ms[2])
    sel_ms = float(call_ms[1])
    step_ms = float(call_ms[4])
    if args.path == "fused":
        dominant, dom_bytes, dom_ms = "hs_decode_step", bytes_step, step_ms
    elif bytes_decode >= bytes_select:
        dominant, dom_bytes, dom_ms = "hs_sparse_decode", bytes_decode, dec_ms
    else:
        dominant, dom_bytes, dom_ms = "hs_select_blocks", bytes_select, sel_ms
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    qheads = w.batch * w.hq

    # ------------------------------------------ decode loop (append + step)
    figures = not args.headline_only and not kc  # the f1-f4 figures use a single level
    want = set(args.figures.split(",")) if figures else set()
    loop = (decode_loop(w, copies[0], pt, stream, args.event_steps, min(args.loop_steps, w.T - 1))
            if args.loop_steps > 0 and "loop" in want else None)
    if loop:
        log("decode loop: %.4f ms per step (append %.4f ms)" % (loop["ms_per_step"],
                                                                  loop["append_ms"]))

    sched = tokens = cache = shared = None
    if "ratio" in want:
        sched = schedule_timing(w, copies, stream, args.event_steps)
        log("ratio %.2f + reserve set: %.4f ms per call, %.0f GB/s" % (
            sched["top_k_ratio"], sched["ms_per_call"], sched["GBps"]))
    if "tokens" in want:
        tokens = token_stage_timing(w, copies, stream, args.event_steps)
        log("token stage: select %.4f ms, attention %.4f ms per call" % (tokens["select_ms"],
                                                                         tokens["decode_ms"]))
    if "cache" in want:
        cache = block_cache_timing(w, stream, args.event_steps)
        log("block cache update: %.4f ms per call (%d slots)" % (cache["ms_per_call"],
                                                                 cache["capacity"]))
    # the headline's inputs are freed before the larger workloads are built
    used_graph, n_inputs = graphs is not None, len(copies)
    del graphs, round_graph, copies, c0, kp0, vp0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    ceiling = stream_ceiling(stream, args.event_steps)
    log("same-box ceilings: copy %.0f GB/s (read + write), read-only reduction %.0f GB/s" % (
        ceiling["copy_GBps"], ceiling["read_GBps"]))
    configs = None
    if "shared" in want:
        shared = shared_selection_timing(stream, args.event_steps)
        log("8 layers, shared selection: %.4f ms per token (%.0f GB/s); own selection per "
            "layer: %.4f ms" % (shared["shared"]["ms_per_token"], shared["shared"]["GBps"],
                                shared["per_layer"]["ms_per_token"]))
        log("selection drift over %d steps: |S_t minus S_t-1| min %d, mean %.1f, max %d" % (
            shared["step_diff"]["steps"], shared["step_diff"]["min"], shared["step_diff"]["mean"],
            shared["step_diff"]["max"]))
    if "configs" in want:
        configs = {}
        for cfg in (1, 2, 4):
            if cfg != args.config:
                configs[str(cfg)] = config_figure(CONFIGS[cfg], stream, args.event_steps)

    # ----------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_seconds)

    result = {
        "metric": "decode query-heads/sec at 128K ctx + effective HBM GB/s as % of MI355X peak",
        "value": qheads / (ms_per_step * 1e-3),
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) bf16 K/V/q with planted needle blocks)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.d, "context": w.T, "summary": w.kind, "block": w.S,
                   "page": w.page_size, "top_k": w.top_k, "window": w.window,
                   "path": args.path, "graph": used_graph, "input_copies": n_inputs,
                   "steps_per_graph": per_round if used_graph else None,
                   "coarse_block": w.coarse_S or None, "top_k_coarse": kc or None},
        "effective_GBps": bytes_step / (ms_per_step * 1e-3) / 1e9,
        "effective_frac_of_peak": bytes_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "bytes_per_step": bytes_step,
        "per_call_ms": {n: float(v) for n, v in zip(names, call_ms)},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(dominant, w.name),
                     "bytes_per_launch": dom_bytes, "avg_ms": dom_ms},
        "separate_calls": {
            "hs_select_blocks": {"GBps": bytes_select / (sel_ms * 1e-3) / 1e9,
                                 "bytes_per_launch": bytes_select, "avg_ms": sel_ms,
                                 "traffic": measured_traffic("hs_select_blocks", w.name)},
            "hs_sparse_decode": {"GBps": bytes_decode / (dec_ms * 1e-3) / 1e9,
                                 "bytes_per_launch": bytes_decode, "avg_ms": dec_ms,
                                 "traffic": measured_traffic("hs_sparse_decode", w.name)}},
        "step_ms_quantiles": step_q,
        "needle_recall": recall,
        "stream_ceiling": ceiling,
        "summary_build": {"ms": build_avg, "GBps": build_bytes / build_avg / 1e6},
        "warm_ms_per_step_single_copy": warm_ms,
        "configs": configs,
        "decode_loop": loop,
        "block_cache": cache,
        "shared_selection": shared,
        "token_stage": tokens,
        "ratio_and_reserve": sched,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def replay_ms(g, stream, reps, inner=4):
    """Per-replay ms of graph `g` on `stream`, one figure per event pair: `reps`
    event pairs, each around `inner` back-to-back replays (so that the host's
    event and launch work overlaps the GPU's rather than adding to short
    replays), after one untimed replay."""
    import numpy as np
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    with torch.cuda.stream(stream):
        g.replay()
        for e0, e1 in evs:
            e0.record(stream)
            for _ in range(inner):
                g.replay()
            e1.record(stream)
    torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) for e0, e1 in evs]) / inner


def timed_graph(body, stream, reps):
    """Mean ms of one replay of a graph captured from body(), over `reps`
    event-timed groups of replays on `stream` after one untimed replay, and
    the per-replay times."""
    import numpy as np
    import torch
    with torch.cuda.stream(stream):
        body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        body()
    torch.cuda.synchronize()
    t = replay_ms(g, stream, reps)
    del g
    return float(t.mean()), t


def stream_ceiling(stream, reps, nbytes=1 << 30):
    """What plain streaming reaches on this GPU, for context: a 1 GiB
    device-to-device copy (read + write) and a read-only row reduction of
    1 GiB (262144 rows of 4 KiB summed, 1 MiB written), each timed as graph
    replays."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    rows = src.view(-1, 1024)
    acc = torch.empty(rows.shape[0], dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    copy_ms, _ = timed_graph(lambda: dst.copy_(src), stream, reps)
    read_ms, _ = timed_graph(lambda: torch.sum(rows, dim=1, out=acc), stream, reps)
    del src, dst, rows, acc
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "copy_ms": copy_ms, "copy_GBps": 2 * nbytes / (copy_ms * 1e-3) / 1e9,
            "read_ms": read_ms, "read_GBps": nbytes / (read_ms * 1e-3) / 1e9}


def config_figure(w, stream, reps, calls=8):
    """One decode step (hs_decode_step: refresh of the growing block of each
    level, selection, attention) of workload w, timed as a graph of `calls`
    back-to-back steps on one copy of the inputs; with algorithmic bytes,
    fraction of the HBM peak, the dominant kernel's measured traffic (from
    profiles/, when taken on the current sources) and needle recall. A step's
    working set that fits the 256 MiB Infinity Cache (the 4K workload) is
    read from the cache after the first call; the record says so."""
    import numpy as np
    import torch

    import hierarchical_sparse_attention_amd as hs
    from synth import device as sdev
    t = time.time()
    log("figure %s: generating inputs" % w.name)
    kp, vp = sdev.make_pools(w)
    kv = hs.KVCache(kp, vp, sdev.page_table_tensor(w), sdev.seq_lens_tensor(w), w.T)
    q = sdev.q_tensor(w)
    fine = hs.Summaries.empty(kv, w.kind, w.S)
    kc = w.top_k_coarse
    coarse = hs.Summaries.empty(kv, "mean", w.coarse_S) if kc else None
    torch.cuda.synchronize()
    hs.hs_build_summaries(kv, fine, 0, stream=stream)
    if kc:
        hs.hs_build_summaries(kv, coarse, 0, stream=stream)
    torch.cuda.synchronize()
    log("figure %s: inputs on device in %.1f s" % (w.name, time.time() - t))
    cap = w.max_selected
    ids = torch.zeros((w.batch, w.hkv, cap), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((w.batch, w.hkv), dtype=torch.int32, device="cuda")
    out = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
    ws = hs.workspace(hs.hs_select_decode_workspace_size(kv, fine, w.hq, w.top_k, w.window, cap,
                                                         coarse, kc), "cuda")
    step = hs.prepare_decode_step(kv, q, fine, w.top_k, w.window, (w.T - 1) // w.S, ids, cnt, out,
                                  ws, stream, coarse, kc)

    def body():
        for _ in range(calls):
            step()

    ms, per = timed_graph(body, stream, reps)
    ms /= calls
    hi, hc = ids.cpu().numpy(), cnt.cpu().numpy()
    nb = step_bytes(w, hi, hc)
    esize = 2 if w.dtype == "bf16" else 4
    row = w.d * 4 if w.kind == "mean" else 2 * w.d * esize
    work = w.units * (w.nb * row + int(hc.max()) * w.S * w.d * esize * 2)
    rec = {"workload": w.name, "config": w.config, "batch": w.batch, "q_heads": w.hq,
           "kv_heads": w.hkv, "head_dim": w.d, "context": w.T, "dtype": w.dtype,
           "summary": w.kind, "block": w.S, "top_k": w.top_k, "window": w.window,
           "coarse_block": w.coarse_S or None, "top_k_coarse": kc or None,
           "entry_point": "hs_decode_step", "calls_per_graph": calls,
           "ms_per_step": ms, "step_ms_p10_p50_p90": [float(np.percentile(per, 10)) / calls,
                                                      float(np.median(per)) / calls,
                                                      float(np.percentile(per, 90)) / calls],
           "query_heads_per_s": w.batch * w.hq / (ms * 1e-3),
           "bytes_per_step": nb["step"], "bytes": {k: v for k, v in nb.items() if k != "step"},
           "GBps": nb["step"] / (ms * 1e-3) / 1e9,
           "frac": nb["step"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "traffic": dominant_traffic(w, nb),
           "head_traffic": measured_traffic("hs_two_level_head", w.name) if kc else None,
           "mean_selected": float(hc.mean()), "needle_recall": needle_recall(w, hi, hc),
           "cache_resident": work < (256 << 20)}
    log("figure %s: %.4f ms per step, %.0f GB/s (%.3f of peak), needle recall %s" % (
        w.name, ms, rec["GBps"], rec["frac"], rec["needle_recall"]))
    del kp, vp, kv, fine, coarse, ws, ids, cnt, out, step
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def decode_loop(w, c, pt, stream, reps, steps=64):
    """Decode-time cache maintenance, timed: the copy's sequences restart
    `steps` tokens short of T; every step appends the next token's K and V
    (hs_append_kv; the rows already cached at that position, so the pools end
    unchanged) and runs hs_decode_step with the refresh of the growing block.
    The whole loop is one captured graph whose first node resets seq_lens."""
    import numpy as np
    import torch

    import hierarchical_sparse_attention_amd as hs
    kv0 = c["kv"]
    t0 = w.T - steps
    sl_init = torch.full((w.batch,), t0, dtype=torch.int32, device="cuda")
    sl = sl_init.clone()
    kv = hs.KVCache(kv0.k_pool, kv0.v_pool, pt, sl, w.T)
    pos = torch.arange(t0, w.T, device="cuda")
    k_new, v_new = [], []
    for pool, dst in ((kv0.k_pool, k_new), (kv0.v_pool, v_new)):
        rows = [pool[pt[b, pos // w.page_size].long(), :, pos % w.page_size] for b in range(w.batch)]
        dst.append(torch.stack(rows, 1).contiguous())  # [steps][B][Hkv][d]
    k_new, v_new = k_new[0], v_new[0]

    def body(with_step):
        sl.copy_(sl_init)
        for i in range(steps):
            hs.hs_append_kv(kv, k_new[i], v_new[i], stream=stream)
            if with_step:
                hs.hs_decode_step(kv, c["q"], c["fine"], w.top_k, w.window, (t0 + i) // w.S,
                                  c["ids"], c["cnt"], c["out"], c["ws_f"], stream=stream)

    out = {}
    for name, with_step in (("loop", True), ("append", False)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            body(with_step)
        torch.cuda.synchronize()
        replay_t = replay_ms(g, stream, reps)
        out[name] = float(replay_t.mean()) / steps
        del g
    assert sl.cpu().tolist() == [w.T] * w.batch
    return {"steps_per_loop": steps, "start_len": t0, "ms_per_step": out["loop"],
            "query_heads_per_s": w.batch * w.hq / (out["loop"] * 1e-3),
            "append_ms": out["append"]}


def schedule_timing(w, copies, stream, reps, reserve=0.01):
    """hs_decode_step with the pages' length-scheduled ratio instead of a fixed
    k (SparDA section 3.2: 5 % at 128K, so k = max(1, int(nb * 0.05))) and a
    seeded random reserve set of `reserve` of each unit's blocks (section 3.4),
    over the rotating input copies; time per call from events around a graph
    of one call per copy, and algorithmic GB/s from the blocks it selected."""
    import numpy as np
    import torch

    import hierarchical_sparse_attention_amd as hs
    ratio = 0.05 if w.T > 32768 else (0.10 if w.T > 16384 else 0.15)
    nb = w.nb
    k = max(1, int(nb * float(np.float32(ratio))))
    r = max(1, int(nb * reserve))
    rng = np.random.default_rng(w.seed + 7)
    forced = np.stack([rng.choice(nb, size=r, replace=False) for _ in range(w.units)])
    forced_t = torch.from_numpy(forced.astype(np.int32).reshape(w.batch, w.hkv, r)).cuda()
    cap = min(nb, k + -(-w.window // w.S) + 1 + r)
    calls, bufs = [], []
    for c in copies:
        ids = torch.zeros((w.batch, w.hkv, cap), dtype=torch.int32, device="cuda")
        cnt = torch.zeros((w.batch, w.hkv), dtype=torch.int32, device="cuda")
        out = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
        n = hs.hs_select_decode_workspace_size(c["kv"], c["fine"], w.hq, w.top_k, w.window, cap,
                                               top_k_ratio=ratio, forced=forced_t)
        ws = hs.workspace(n, "cuda")
        bufs.append((ids, cnt, out, ws))
        calls.append(lambda c=c, ids=ids, cnt=cnt, out=out, ws=ws: hs.hs_decode_step(
            c["kv"], c["q"], c["fine"], w.top_k, w.window, (w.T - 1) // w.S, ids, cnt, out, ws,
            stream=stream, top_k_ratio=ratio, forced=forced_t))
    with torch.cuda.stream(stream):
        for call in calls:
            call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for call in calls:
            call()
    torch.cuda.synchronize()
    replay_t = replay_ms(g, stream, reps)
    ms = float(replay_t.mean()) / len(calls)
    ids, cnt = bufs[0][0].cpu().numpy(), bufs[0][1].cpu().numpy()
    lens = w.seq_lens_array()
    esize = 2 if w.dtype == "bf16" else 4
    tokens = sum(int(np.minimum(w.S, lens[b] - ids[b, g, :cnt[b, g]].astype(np.int64) * w.S).sum())
                 for b in range(w.batch) for g in range(w.hkv))
    row = w.d * 4 if w.kind == "mean" else 2 * w.d * esize
    nbytes = (tokens * w.d * esize * 2 + w.units * w.nb * row + w.units * (w.S * w.d * esize + row)
              + w.batch * w.hq * w.d * (esize + 4) + int(cnt.sum()) * 4)
    return {"top_k_ratio": ratio, "k": k, "reserve_blocks": r, "max_selected": cap,
            "mean_selected": float(cnt.mean()), "ms_per_call": ms,
            "bytes_per_call": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9}


def token_stage_timing(w, copies, stream, reps, k_tok=1024, window=512):
    """The token-level second stage on top of each copy's block selection (the
    ids the timed step wrote): hs_select_tokens keeps the top `k_tok` tokens of
    the selected blocks plus the `window` last tokens, then hs_sparse_decode
    with block size 1 attends over them. Each call is timed with events around
    a graph of one call per copy."""
    import numpy as np
    import torch

    import hierarchical_sparse_attention_amd as hs
    ms = w.max_selected
    max_tok = min(ms * w.S, k_tok) + min(window, w.T)
    sel, dec, bufs = [], [], []
    for c in copies:
        tok = torch.zeros((w.batch, w.hkv, max_tok), dtype=torch.int32, device="cuda")
        tcnt = torch.zeros((w.batch, w.hkv), dtype=torch.int32, device="cuda")
        out = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
        ws_t = hs.workspace(hs.hs_select_tokens_workspace_size(c["kv"], w.hq, w.S, ms, k_tok,
                                                               window, max_tok), "cuda")
        ws_d = hs.workspace(hs.hs_decode_workspace_size(c["kv"], w.hq, 1, max_tok), "cuda")
        bufs.append((tok, tcnt, out, ws_t, ws_d))
        sel.append(lambda c=c, tok=tok, tcnt=tcnt, ws_t=ws_t: hs.hs_select_tokens(
            c["kv"], c["q"], w.S, c["ids"], c["cnt"], k_tok, window, tok, tcnt, ws_t,
            stream=stream))
        dec.append(lambda c=c, tok=tok, tcnt=tcnt, out=out, ws_d=ws_d: hs.hs_sparse_decode(
            c["kv"], c["q"], 1, tok, tcnt, out, ws_d, stream=stream))
    res = {}
    for name, calls in (("select_ms", sel), ("decode_ms", dec)):
        with torch.cuda.stream(stream):
            for call in calls:
                call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for call in calls:
                call()
        torch.cuda.synchronize()
        replay_t = replay_ms(g, stream, reps)
        res[name] = float(replay_t.mean()) / len(calls)
        del g
    esize = 2 if w.dtype == "bf16" else 4
    cnt = copies[0]["cnt"].cpu().numpy()
    ids = copies[0]["ids"].cpu().numpy()
    lens = w.seq_lens_array()
    cand = sum(int(np.minimum(w.S, lens[b] - ids[b, g, :cnt[b, g]].astype(np.int64) * w.S).sum())
               for b in range(w.batch) for g in range(w.hkv))
    kept = int(bufs[0][1].cpu().numpy().sum())
    sel_bytes = cand * w.d * esize + w.batch * w.hq * w.d * esize + int(cnt.sum()) * 4 + kept * 4
    dec_bytes = kept * w.d * esize * 2 + w.batch * w.hq * w.d * (esize + 4) + kept * 4
    res.update({"k_tokens": k_tok, "window": window, "candidate_tokens": cand,
                "kept_tokens": kept, "select_bytes": sel_bytes, "decode_bytes": dec_bytes,
                "select_GBps": sel_bytes / (res["select_ms"] * 1e-3) / 1e9,
                "select_frac": sel_bytes / (res["select_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "decode_GBps": dec_bytes / (res["decode_ms"] * 1e-3) / 1e9,
                "decode_frac": dec_bytes / (res["decode_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "select_traffic": measured_traffic("hs_select_tokens", w.name),
                "decode_traffic": measured_traffic("hs_sparse_decode_tokens", w.name)})
    return res


def block_cache_timing(w, stream, reps, steps=16, keep=0.85):
    """hs_block_cache_update at the workload's shape (B * Hkv units, max_selected
    ids, 4 x max_selected slots) over `steps` seeded drifting selections: each
    step keeps about `keep` of a unit's previous blocks (the pages report 80-90 %
    overlap between consecutive steps) and draws the rest anew. One captured
    graph: the cache is refilled with -1, then the steps run in order."""
    import numpy as np
    import torch

    import hierarchical_sparse_attention_amd as hs
    ms, units = w.max_selected, w.units
    rng = np.random.default_rng(w.seed + 99)
    ids = np.full((steps, units, ms), -1, np.int32)
    cnt = np.zeros((steps, units), np.int32)
    for u in range(units):
        cur = np.sort(rng.choice(w.nb, size=ms - 1, replace=False))
        for t in range(steps):
            if t:
                kept = cur[rng.random(len(cur)) < keep]
                pool = np.setdiff1d(np.arange(w.nb), kept)
                cur = np.sort(np.concatenate([kept, rng.choice(pool, size=ms - 1 - len(kept),
                                                               replace=False)]))
            ids[t, u, :len(cur)] = cur
            cnt[t, u] = len(cur)
    d_ids = torch.from_numpy(ids).cuda()
    d_cnt = torch.from_numpy(cnt).cuda()
    cache = hs.BlockCache.empty(units, 4 * ms)
    slot_of = torch.empty((units, ms), dtype=torch.int32, device="cuda")
    miss = torch.empty_like(slot_of)
    stats = torch.empty((steps, units, 3), dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        cache.slot_block.fill_(-1)
        cache.slot_stamp.fill_(-1)
        for t in range(steps):
            hs.hs_block_cache_update(cache, t, d_ids[t], d_cnt[t], slot_of, miss, stats[t],
                                     stream=stream)
    torch.cuda.synchronize()
    replay_t = replay_ms(g, stream, reps)
    ms_call = float(replay_t.mean()) / steps
    st = stats.cpu().numpy()[1:]  # steps after the first (cold) one
    return {"capacity": 4 * ms, "units": units, "steps": steps, "ms_per_call": ms_call,
            "mean_overlap": float(1.0 - st[:, :, 2].sum() / st[:, :, :2].sum()),
            "miss_rate": float(st[:, :, 1].sum() / st[:, :, :2].sum())}


def shared_selection_timing(stream, reps):
    """The 8-layer shared-selection workload (16 sequences of 64K tokens, GQA
    32/8, d 128, bf16, mean summaries over 64-token pages, k 102, W 512, a
    seeded page permutation), one decode token through all 8 layers, each
    layer's K/V in its own pools. Shared: layer 0 runs hs_decode_step (refresh,
    selection, attention) and layers 1-7 run hs_sparse_decode over the same
    ids (SparDA section 3.3). Per layer, for contrast: every layer runs
    hs_decode_step on its own summaries. Each variant is one captured graph,
    timed with events."""
    import numpy as np
    import torch

    import hierarchical_sparse_attention_amd as hs
    from synth import device as sdev
    from synth.workloads import CONFIGS

    w = CONFIGS[5]
    esize = 2 if w.dtype == "bf16" else 4
    t = time.time()
    pt = sdev.page_table_tensor(w)
    sl = sdev.seq_lens_tensor(w)
    cap = w.max_selected
    last_block = (w.T - 1) // w.S
    layers = []
    for layer in range(w.layers):
        kp, vp = sdev.make_pools(w, layer)
        kv = hs.KVCache(kp, vp, pt, sl, w.T)
        fine = hs.Summaries.empty(kv, w.kind, w.S)
        L = dict(kv=kv, fine=fine, q=sdev.q_tensor(w, layer, 0),
                 ids=torch.zeros((w.batch, w.hkv, cap), dtype=torch.int32, device="cuda"),
                 cnt=torch.zeros((w.batch, w.hkv), dtype=torch.int32, device="cuda"),
                 out=torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda"),
                 ws_f=hs.workspace(hs.hs_select_decode_workspace_size(
                     kv, fine, w.hq, w.top_k, w.window, cap), "cuda"),
                 ws_d=hs.workspace(hs.hs_decode_workspace_size(kv, w.hq, w.S, cap), "cuda"))
        layers.append(L)
    torch.cuda.synchronize()  # pools filled on torch's stream before the builds on `stream`
    for L in layers:
        hs.hs_build_summaries(L["kv"], L["fine"], 0, stream=stream)
    torch.cuda.synchronize()
    log("shared selection: %d layers on device in %.1f s" % (w.layers, time.time() - t))
    L0 = layers[0]

    def shared():
        hs.hs_decode_step(L0["kv"], L0["q"], L0["fine"], w.top_k, w.window, last_block,
                          L0["ids"], L0["cnt"], L0["out"], L0["ws_f"], stream=stream)
        for L in layers[1:]:
            hs.hs_sparse_decode(L["kv"], L["q"], w.S, L0["ids"], L0["cnt"], L["out"], L["ws_d"],
                                stream=stream)

    def own():
        for L in layers:
            hs.hs_decode_step(L["kv"], L["q"], L["fine"], w.top_k, w.window, last_block,
                              L["ids"], L["cnt"], L["out"], L["ws_f"], stream=stream)

    lens = w.seq_lens_array()

    def decode_bytes(ids, cnt):
        tok = sum(int(np.minimum(w.S, lens[b] - ids[b, g, :cnt[b, g]].astype(np.int64) * w.S).sum())
                  for b in range(w.batch) for g in range(w.hkv))
        return tok * w.d * esize * 2 + w.batch * w.hq * w.d * (esize + 4) + int(cnt.sum()) * 4

    row = w.d * 4 if w.kind == "mean" else 2 * w.d * esize
    select_bytes = w.units * w.nb * row + w.units * (w.S * w.d * esize + row)
    res = {"workload": w.name, "layers": w.layers, "batch": w.batch, "q_heads": w.hq,
           "kv_heads": w.hkv, "context": w.T, "block": w.S, "top_k": w.top_k,
           "window": w.window, "page_table": "seeded permutation"}
    for name, body in (("shared", shared), ("per_layer", own)):
        with torch.cuda.stream(stream):
            body()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            body()
        torch.cuda.synchronize()
        replay_t = replay_ms(g, stream, reps)
        ms = float(replay_t.mean())
        del g
        if name == "shared":
            b0 = decode_bytes(L0["ids"].cpu().numpy(), L0["cnt"].cpu().numpy())
            nbytes = select_bytes + w.layers * b0
            mean_sel = float(L0["cnt"].float().mean())
        else:
            nbytes = sum(select_bytes + decode_bytes(L["ids"].cpu().numpy(), L["cnt"].cpu().numpy())
                         for L in layers)
            mean_sel = float(np.mean([float(L["cnt"].float().mean()) for L in layers]))
        res[name] = {"ms_per_token": ms, "query_heads_per_s": w.batch * w.hq / (ms * 1e-3),
                     "bytes_per_token": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9,
                     "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "mean_selected": mean_sel}
    # HBM bytes per launch of the two kernels (layer 0's step, the other layers'
    # decode), when a matching rocprofv3 summary exists
    res["shared"]["traffic"] = {k: measured_traffic(k, w.name)
                                for k in ("hs_decode_step", "hs_sparse_decode")}
    # the selection's drift: layer-0 selections over the workload's decode steps
    # (query q_t = 0.9 q_{t-1} + 0.44 n_t), |S_t minus S_t-1| per unit, untimed
    ws_s = hs.workspace(hs.hs_select_workspace_size(L0["kv"], L0["fine"], w.hq, w.top_k,
                                                    w.window, cap), "cuda")
    ids_t = torch.zeros_like(L0["ids"])
    cnt_t = torch.zeros_like(L0["cnt"])
    prev, diffs = None, []
    for t in range(w.steps):
        hs.hs_select_blocks(L0["kv"], sdev.q_tensor(w, 0, t), L0["fine"], w.top_k, w.window,
                            ids_t, cnt_t, ws_s)
        ids, cnt = ids_t.cpu().numpy(), cnt_t.cpu().numpy()
        cur = [set(ids[b, g, :cnt[b, g]].tolist()) for b in range(w.batch) for g in range(w.hkv)]
        if prev is not None:
            diffs.append([len(c - p_) for c, p_ in zip(cur, prev)])
        prev = cur
    d = np.array(diffs, dtype=np.float64)
    res["step_diff"] = {"steps": w.steps, "min": int(d.min()), "mean": float(d.mean()),
                        "max": int(d.max()), "mean_selected": float(np.mean([len(c) for c in prev]))}
    del layers, L0
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, seconds):
    """The CPU oracle on this host, the same workload, in two parts like the
    GPU's: the summary build (prefill phase) and one decode step (selection
    from those summaries + attention, over every unit of the batch). Input
    generation and widening are excluded. Timed at 1 thread (units one after
    another on a sample, extrapolated to the full batch) and at N threads, N =
    the host's available cores, running the full batch's units concurrently
    (the oracle's C calls release the GIL), each for about `seconds`."""
    import platform
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth

    host_cores = len(os.sched_getaffinity(0))
    units = [(b, g) for b in range(w.batch) for g in range(w.hkv)]
    t = time.time()
    prep = []
    for b, g in units:
        q = synth.widen(w.q(), w.dtype)[b, g * w.G:(g + 1) * w.G]
        prep.append([q, synth.widen(w.k_unit(0, b, g), w.dtype),
                     synth.widen(w.v_unit(0, b, g), w.dtype), None])
    log("cpu baseline: %d units widened in %.1f s; %d host cores" % (len(units), time.time() - t,
                                                                    host_cores))

    def build(i):
        prep[i][3] = oracle.summarize(prep[i][1], w.S, w.kind)

    def step(i):
        q, K, V, (a, c) = prep[i]
        sel = oracle.select_unit(q, K, w.T, w.kind, w.S, w.top_k, w.window, summaries=(a, c, None, None))
        oracle.attend_unit(q, K, V, w.T, sel.ids, w.S)

    def one_thread(fn):
        """Seconds per unit: units one after another, cycling, for ~seconds."""
        n, t0 = 0, time.perf_counter()
        while n < len(units) and (n == 0 or time.perf_counter() - t0 < seconds):
            fn(n)
            n += 1
        return (time.perf_counter() - t0) / n, n

    def n_threads(fn, ex):
        """Seconds per full batch (every unit once, N threads), repeated for ~seconds."""
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < seconds:
            list(ex.map(fn, range(len(units))))
            reps += 1
        return (time.perf_counter() - t0) / reps, reps

    with ThreadPoolExecutor(max_workers=host_cores) as ex:
        list(ex.map(build, range(len(units))))  # every unit's summaries, untimed
        b1, nb1 = one_thread(build)
        bn, rbn = n_threads(build, ex)
        s1, ns1 = one_thread(step)
        sn, rsn = n_threads(step, ex)
    qh = w.batch * w.hq
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    step1 = s1 * len(units)
    log("cpu baseline: step %.3f s at 1 thread (from %d units), %.3f s at %d threads; summary "
        "build %.3f s / %.3f s" % (step1, ns1, sn, host_cores, b1 * len(units), bn))
    return {"value": qh / sn, "unit": "query-heads/s", "cores": host_cores, "kind": "oracle",
            "sample": "the full batch (%d units of %d query heads), selection from the oracle's "
                      "own summaries + attention per unit, %d repetitions on %d threads (%.1f s); "
                      "1-thread figure from %d units run one after another" % (
                          len(units), w.G, rsn, host_cores, sn * rsn, ns1),
            "host_cores": host_cores, "cpu_model": model,
            "threads_1": {"s_per_step": step1, "query_heads_per_s": qh / step1,
                          "s_per_unit": s1, "units_timed": ns1,
                          "summary_build_s": b1 * len(units)},
            "threads_N": {"threads": host_cores, "s_per_step": sn, "query_heads_per_s": qh / sn,
                          "steps_timed": rsn, "summary_build_s": bn},
            "excluded": "input generation and widening to float64"}

if __name__ == "__main__":
    main()
