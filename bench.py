#!/usr/bin/env python3
"""Benchmark of the rotated INT2 KV-cache hot path on one MI355X.

One step runs the whole hot path once per layer through kvq_append_decode:
it encodes one new bf16 key/value token per sequence (centre, rotate, clip,
INT2 group RTN, pack into the paged cache) and runs single-token attention
over the updated INT2 cache (rotated query, split-K online softmax,
log-sum-exp merge, inverse value rotation).  --separate-calls runs the same
step as kvq_append followed by kvq_decode_attn.

Default workload: 36 layers x batch 16 of Qwen3-8B-shaped attention (32
query / 8 KV heads, head_dim 128), 16K tokens of prior context per sequence,
paged blocks of 16, group 128, clip 0.9.  All inputs are seeded synthetic
data resident in HBM before timing starts.  Each step is captured once as a
HIP graph and replayed.  Prints one JSON line.
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

METRIC = "INT2 decode-attention cache GB/s (% of HBM peak) and tokens/s; append Mtok/s"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_36l_b16_ctx16k_stream")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's CPU time for the cpu_baseline leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying graphs")
    ap.add_argument("--no-windows", action="store_true",
                    help="skip the second pass with BF16 sink/recent windows")
    ap.add_argument("--separate-calls", action="store_true",
                    help="kvq_append + kvq_decode_attn per layer instead of kvq_append_decode")
    ap.add_argument("--no-folded", action="store_true",
                    help="skip the pass with the value rotation folded into W_V/W_O (rot_v NULL)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill comparison (the prompts encoded with both rotations, "
                         "with R_V folded, and unrotated)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the cold long-context decode leg (128K batch 1; ragged 1K-32K batch 64)")
    ap.add_argument("--long-reps", type=int, default=24,
                    help="decode calls timed per long-context workload (at least one per cache copy)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the measurement, run a plain fp32 copy kernel (y = -x) over this "
                         "many MiB three times: the reference for HBM byte counters")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_kernel_traffic.json")


def measured_traffic(workload: str, kernel: str, grid_threads: int):
    """HBM bytes per scan launch from the committed counter summary, or None if
    it was taken on another workload, kernel or grid, or the kernel's sources
    changed since."""
    from rotated_int2_kv_kvq_amd.traffic import kernel_source_hash
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("workload") != workload or rec.get("kernel") != kernel
            or rec.get("grid_threads") != grid_threads
            or rec.get("source_sha256") != kernel_source_hash()):
        return None
    return round(float(rec["traffic_bytes"]))


def cache_bytes_per_token_head(group: int) -> int:
    """Algorithmic INT2 cache bytes decode reads per (token, KV head):
    K and V codes (2 x 32 B) plus one fp16 (scale, zero) pair per group for each."""
    return 2 * (128 // 4) + 2 * (128 // group) * 4


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rotated_int2_kv_kvq_amd as kvq
    from workload import WORKLOADS, key_mean, kv_for_sequence, make_static, query_for, scaled

    dev = "cuda"
    kvq.lib()
    total_steps = args.warmup + args.steps
    w0 = WORKLOADS[args.workload]
    w = scaled(w0, steps=max(w0.steps, total_steps))
    st = make_static(w)
    L, B, Hq, Hkv, d = w.layers, w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    pb = kvq.page_bytes(d, w.group)
    table = torch.from_numpy(st.block_table).to(dev)
    ctx0 = st.ctx_lens.astype(np.int64)

    # ---------------------------------------------------------------- build the cache
    pages, mus, rks, rvs, wins = [], [], [], [], []
    t_bulk = 0.0
    n_bulk = 0
    for layer in range(L):
        pages.append(torch.empty(st.num_blocks, Hkv, pb, dtype=torch.uint8, device=dev))
        mus.append(key_mean(w, st, layer, device=dev).contiguous())
        rks.append(torch.from_numpy(st.rot_k[layer]).to(dev).contiguous())
        rvs.append(torch.from_numpy(st.rot_v[layer]).to(dev).contiguous())
        by_len = {}
        for b, n in enumerate(ctx0):
            by_len.setdefault(int(n), []).append(b)
        for n, seqs in by_len.items():
            kv = [kv_for_sequence(w, st, layer, b, 0, n, dev) for b in seqs]
            k = torch.stack([x[0] for x in kv]).contiguous()
            v = torch.stack([x[1] for x in kv]).contiguous()
            del kv
            tab = table.index_select(0, torch.as_tensor(seqs, device=dev)).contiguous()
            sp = torch.zeros(len(seqs), dtype=torch.int32, device=dev)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            kvq.append(pages[layer], tab, sp, k, v, mus[layer], rks[layer], rvs[layer], w.group,
                       w.clip_k, w.clip_v)
            torch.cuda.synchronize()
            t_bulk += time.perf_counter() - t0
            n_bulk += len(seqs) * n
            if not args.no_windows:
                # BF16 windows of the prompt: its sinks and its last 256 tokens
                if len(wins) == layer:
                    wins.append(kvq.new_window(B, Hkv, dev))
                for i, b in enumerate(seqs):
                    wb = wins[layer][b:b + 1]
                    ns = min(n, kvq.WINDOW_SINK)
                    r0 = max(ns, n - kvq.WINDOW_RECENT)
                    for a0, a1 in ((0, ns), (r0, n)):
                        if a1 > a0:
                            kvq.window_write(wb, torch.full((1,), a0, dtype=torch.int32,
                                                            device=dev),
                                             k[i:i + 1, a0:a1].contiguous(),
                                             v[i:i + 1, a0:a1].contiguous())
            del k, v
        print(f"[bench] layer {layer} cache built", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- per-step inputs
    qs, kn, vn, spos, ctxs, maxc = [], [], [], [], [], []
    new_kv = []  # [layer] -> (k, v) of shape [B][total_steps][Hkv][d]
    for layer in range(L):
        kv = [kv_for_sequence(w, st, layer, b, int(ctx0[b]), total_steps, dev) for b in range(B)]
        new_kv.append((torch.stack([x[0] for x in kv]), torch.stack([x[1] for x in kv])))
    for step in range(total_steps):
        qs.append([query_for(w, layer, step, dev).contiguous() for layer in range(L)])
        kn.append([new_kv[layer][0][:, step:step + 1].contiguous() for layer in range(L)])
        vn.append([new_kv[layer][1][:, step:step + 1].contiguous() for layer in range(L)])
        spos.append(torch.from_numpy((ctx0 + step).astype(np.int32)).to(dev))
        ctxs.append(torch.from_numpy((ctx0 + step + 1).astype(np.int32)).to(dev))
        maxc.append(int(ctx0.max()) + step + 1)
    max_ctx_all = maxc[-1]
    ws = torch.empty(kvq.decode_workspace_bytes(B, Hq, Hkv, max_ctx_all, d), dtype=torch.uint8,
                     device=dev)
    outs = [torch.empty(B, Hq, d, dtype=torch.float32, device=dev) for _ in range(L)]
    sm_scale = 1.0 / math.sqrt(d)

    def run_step(step):
        for layer in range(L):
            if args.separate_calls:
                kvq.append(pages[layer], table, spos[step], kn[step][layer], vn[step][layer],
                           mus[layer], rks[layer], rvs[layer], w.group, w.clip_k, w.clip_v)
                kvq.decode(pages[layer], table, ctxs[step], maxc[step], qs[step][layer],
                           rks[layer], rvs[layer], w.group, sm_scale, out=outs[layer],
                           workspace=ws)
            else:
                kvq.append_decode(pages[layer], table, spos[step], ctxs[step], maxc[step],
                                  kn[step][layer], vn[step][layer], mus[layer], qs[step][layer],
                                  rks[layer], rvs[layer], w.group, w.clip_k, w.clip_v, sm_scale,
                                  out=outs[layer], workspace=ws)

    graphs = []
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        for step in range(total_steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                run_step(step)
            graphs.append(g)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        # capture does not execute: the cache still holds only the prior context

    def step_fn(step):
        if graphs:
            graphs[step].replay()
        else:
            run_step(step)

    # ---------------------------------------------------------------- timed steps
    for step in range(args.warmup):
        step_fn(step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for step in range(args.warmup, total_steps):
        step_fn(step)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    step_ms = gpu_ms / args.steps
    per_tok_head = cache_bytes_per_token_head(w.group)
    bytes_steps = sum(int((ctx0 + s + 1).sum()) * Hkv * per_tok_head * L
                      for s in range(args.warmup, total_steps))
    value = bytes_steps / (gpu_ms * 1e-3) / 1e9
    assert all(torch.isfinite(o).all().item() for o in outs)

    # ---------------------------------------------------------------- per-kernel event timing
    # The decode stages are launched separately, each layer with its own
    # workspace; the split kernels of all layers run back to back between one
    # pair of events, and so do the single-token appends.  Every launch is
    # queued behind a GPU sleep so that host launch latency never falls inside
    # an event interval.  Where the plan builds the query operand inside the
    # scan, PREPARE and SPLITS together are that one launch, the step's scan
    # kernel (whose launch in the step also encodes the new tokens, in 128
    # workgroups after the splits); otherwise PREPARE runs untimed and SPLITS
    # alone is timed.
    last = total_steps - 1
    plan = kvq.decode_plan(B, Hq, Hkv, maxc[last])
    scan_stages = (kvq.STAGE_PREPARE | kvq.STAGE_SPLITS if plan["operand_in_scan"]
                   else kvq.STAGE_SPLITS)
    scan_kernel = scan_kernel_name(w.group, plan["operand_in_scan"])
    # threads of the timed launch: a 256-thread workgroup per split, or, where
    # the scan builds its own operand at group 128, 512 threads per pair of
    # consecutive splits
    S = plan["num_splits"]
    pairs = plan["operand_in_scan"] and w.group == 128
    scan_threads = 256 * (2 * ((S + 1) // 2) if pairs else S) * Hkv * ((Hq // Hkv + 3) // 4) * B
    wss = [ws] + [torch.empty_like(ws) for _ in range(L - 1)]
    split_ms, app_ms = [], []
    for rep in range(4):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(50_000_000)
        s0, s1, a0, a1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
        if not plan["operand_in_scan"]:
            for layer in range(L):
                kvq.decode(pages[layer], table, ctxs[last], maxc[last], qs[last][layer],
                           rks[layer], rvs[layer], w.group, sm_scale, out=outs[layer],
                           workspace=wss[layer], stages=kvq.STAGE_PREPARE)
        s0.record()
        for layer in range(L):
            kvq.decode(pages[layer], table, ctxs[last], maxc[last], qs[last][layer], rks[layer],
                       rvs[layer], w.group, sm_scale, out=outs[layer], workspace=wss[layer],
                       stages=scan_stages)
        s1.record()
        for layer in range(L):
            kvq.decode(pages[layer], table, ctxs[last], maxc[last], qs[last][layer], rks[layer],
                       rvs[layer], w.group, sm_scale, out=outs[layer], workspace=wss[layer],
                       stages=kvq.STAGE_MERGE)
        a0.record()
        for layer in range(L):
            # re-append the last step's token: same slot, same bytes
            kvq.append(pages[layer], table, spos[last], kn[last][layer], vn[last][layer],
                       mus[layer], rks[layer], rvs[layer], w.group, w.clip_k, w.clip_v)
        a1.record()
        torch.cuda.synchronize()
        if rep == 0:
            continue
        split_ms.append(s0.elapsed_time(s1) / L)
        app_ms.append(a0.elapsed_time(a1) / L)
    del wss
    # host copies of the first and last layers' caches as the main pass left
    # them (later passes re-encode the prompt), for the CPU baseline
    host_pages = {0: pages[0].cpu(), L - 1: pages[L - 1].cpu()}
    split_avg_ms = float(np.mean(split_ms))
    app_avg_ms = float(np.mean(app_ms))
    split_bytes = int((ctx0 + last + 1).sum()) * Hkv * per_tok_head
    achieved = split_bytes / (split_avg_ms * 1e-3) / 1e9

    # ---------------------------------------------------------------- BF16 windows pass
    # The same steps again through kvq_append_decode_window: each step's token
    # enters the recent window and the token it displaces (position p - 256)
    # is encoded into the INT2 body (the same bytes the first pass wrote there).
    win_line = None
    if not args.no_windows:
        def run_wstep(step):
            for layer in range(L):
                kvq.append_decode_window(pages[layer], table, wins[layer], spos[step], ctxs[step],
                                         maxc[step], kn[step][layer], vn[step][layer], mus[layer],
                                         qs[step][layer], rks[layer], rvs[layer], w.group,
                                         w.clip_k, w.clip_v, sm_scale, out=outs[layer],
                                         workspace=ws)
        wgraphs = []
        if not args.no_graph:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            for step in range(total_steps):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    run_wstep(step)
                wgraphs.append(g)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
        for step in range(args.warmup):
            wgraphs[step].replay() if wgraphs else run_wstep(step)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for step in range(args.warmup, total_steps):
            wgraphs[step].replay() if wgraphs else run_wstep(step)
        e1.record()
        torch.cuda.synchronize()
        w_ms = e0.elapsed_time(e1)
        assert all(torch.isfinite(o).all().item() for o in outs)
        body_b = win_b = 0
        for s_ in range(args.warmup, total_steps):
            for n in (ctx0 + s_ + 1):
                nw = min(int(n), kvq.WINDOW_SINK) + min(max(int(n) - kvq.WINDOW_SINK, 0),
                                                        kvq.WINDOW_RECENT)
                body_b += max(int(n) - nw, 0) * Hkv * per_tok_head * L
                win_b += nw * Hkv * 2 * d * 2 * L
        win_line = {
            "step_call": "kvq_append_decode_window",
            "sink": kvq.WINDOW_SINK, "recent": kvq.WINDOW_RECENT,
            "ms_per_step": round(w_ms / args.steps, 4),
            "value": round((body_b + win_b) / (w_ms * 1e-3) / 1e9, 2),
            "unit": "GB/s (INT2 body + BF16 window bytes read)",
            "decode_tokens_per_s": round(B * args.steps / (w_ms * 1e-3), 1),
        }
        del wgraphs


    # ---------------------------------------------------------------- folded value rotation
    # The pages' deployment form: R_V folded into W_V and W_O, so the library
    # gets rot_v = NULL.  The prompt is re-encoded that way (values as given;
    # the bulk append rate of this form), then the same steps are replayed.
    fold_line = None
    if not args.no_folded:
        t_fold = 0.0
        n_fold = 0
        by_len = {}
        for b, n in enumerate(ctx0):
            by_len.setdefault(int(n), []).append(b)
        for layer in range(L):
            for n, seqs in by_len.items():
                kv = [kv_for_sequence(w, st, layer, b, 0, n, dev) for b in seqs]
                k = torch.stack([x[0] for x in kv]).contiguous()
                v = torch.stack([x[1] for x in kv]).contiguous()
                del kv
                tab = table.index_select(0, torch.as_tensor(seqs, device=dev)).contiguous()
                sp = torch.zeros(len(seqs), dtype=torch.int32, device=dev)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                kvq.append(pages[layer], tab, sp, k, v, mus[layer], rks[layer], None, w.group,
                           w.clip_k, w.clip_v)
                torch.cuda.synchronize()
                t_fold += time.perf_counter() - t0
                n_fold += len(seqs) * n
                del k, v

        def run_fstep(step):
            for layer in range(L):
                kvq.append_decode(pages[layer], table, spos[step], ctxs[step], maxc[step],
                                  kn[step][layer], vn[step][layer], mus[layer], qs[step][layer],
                                  rks[layer], None, w.group, w.clip_k, w.clip_v, sm_scale,
                                  out=outs[layer], workspace=ws)
        fgraphs = []
        if not args.no_graph:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            for step in range(total_steps):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    run_fstep(step)
                fgraphs.append(g)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
        for step in range(args.warmup):
            fgraphs[step].replay() if fgraphs else run_fstep(step)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for step in range(args.warmup, total_steps):
            fgraphs[step].replay() if fgraphs else run_fstep(step)
        e1.record()
        torch.cuda.synchronize()
        f_ms = e0.elapsed_time(e1)
        assert all(torch.isfinite(o).all().item() for o in outs)
        fold_line = {
            "step_call": "kvq_append_decode with rot_v NULL (value rotation folded into W_V/W_O)",
            "ms_per_step": round(f_ms / args.steps, 4),
            "value": round(bytes_steps / (f_ms * 1e-3) / 1e9, 2),
            "unit": "GB/s",
            "hbm_frac": round(bytes_steps / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_tokens_per_s": round(B * args.steps / (f_ms * 1e-3), 1),
            "append_bulk_mtok_s": round(n_fold / t_fold / 1e6, 3) if t_fold else None,
        }
        del fgraphs

    # ---------------------------------------------------------------- prefill overhead
    prefill = None
    if not args.no_prefill:
        prefill = prefill_leg(w, st, table, pages[0], mus[0], rks[0], rvs[0], dev)

    # ---------------------------------------------------------------- long contexts, cold
    long_line = None
    if not args.no_long:
        del pages, wins, new_kv, kn, vn
        pages = None
        torch.cuda.empty_cache()
        long_line = {name: long_context_leg(name, args.long_reps)
                     for name in LONG_WORKLOADS}

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        sample_steps = sorted({args.warmup, args.warmup + args.steps // 2, total_steps - 1})
        samples = [(layer, step, host_pages[layer], ctxs[step].cpu(), qs[step][layer].cpu())
                   for layer in sorted(host_pages) for step in sample_steps]
        cpu = cpu_baseline(w, st, samples, table, per_tok_head, args.cpu_seconds, sm_scale)

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        x = torch.randn(n, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x {4 * n} bytes read and written", file=sys.stderr,
              flush=True)
        del x, y

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w0.name, "layers": L, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
            "head_dim": d, "prior_ctx": int(ctx0.max()), "group": w.group, "block": 16,
            "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype, "clip": w.clip_k,
            "cache": f"INT2 + fp16 scale/zero per {w.group} ({per_tok_head} B per token-head)",
            "launch": "eager" if args.no_graph else "hipGraph per step", "parallelism": "none",
            "step_call": ("kvq_append + kvq_decode_attn" if args.separate_calls
                          else "kvq_append_decode"),
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(B * args.steps / (gpu_ms * 1e-3), 1),
        "append_decode_mtok_s": round(B / (app_avg_ms * 1e-3) / 1e6, 4),
        "append_bulk_mtok_s": round(n_bulk / t_bulk / 1e6, 3) if t_bulk else None,
        "append_avg_us": round(app_avg_ms * 1e3, 2),
        "split_kernel_avg_us": round(split_avg_ms * 1e3, 2),
        "wall_s": round(wall, 3),
        "roofline": {
            "kernel": f"{scan_kernel} (decode split-K scan)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w0.name, scan_kernel, scan_threads),
            "algorithmic_bytes": split_bytes,
            "grid_threads": scan_threads,
        },
        "cpu_baseline": cpu,
        "bits_per_element": bits_per_element(w.group),
        "prefill": prefill,
        "context": pages_context(w, ctx0, per_tok_head, prefill),
        "windows": win_line,
        "folded": fold_line,
        "long_context": long_line,
    }
    print(json.dumps(line), flush=True)


def scan_kernel_name(group, operand_in_scan, windows=False, wide=False):
    """The scan kernel's name as rocprofv3 prints it: split_kernel<G, wide
    descriptor, windows, operand built in the scan>."""
    b = lambda x: "true" if x else "false"  # noqa: E731
    return (f"split_kernel<{1 if group == 128 else 2}, {b(wide)}, {b(windows)}, "
            f"{b(operand_in_scan)}>")


def cpu_baseline(w, st, samples, table, per_tok_head, budget_s, sm_scale):
    """The float64 oracle's decode on the host, in cache GB/s, over a bounded
    sample of the timed work: each (layer, step) of `samples` gets an equal
    share of the time budget and decodes (sequence, KV head) pairs in order
    until its share is spent.  First with one BLAS thread, then (under
    "all_cores") with one per host core, at most 16, for two thirds of the
    budget."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        res = _cpu_baseline(O, w, st, samples, table, per_tok_head, budget_s, sm_scale, 1)
    n = min(os.cpu_count() or 1, 16)
    if n > 1:
        with threadpool_limits(n):
            res["all_cores"] = _cpu_baseline(O, w, st, samples, table, per_tok_head,
                                             budget_s * 2 / 3, sm_scale, n)
    res["cpu_model"] = _cpu_model()
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(O, w, st, samples, table, per_tok_head, budget_s, sm_scale, threads):
    import numpy as np
    tab = table.cpu()
    Hkv, Hg = w.num_kv_heads, w.num_q_heads // w.num_kv_heads
    done_bytes = 0
    pairs = 0
    share = budget_s / len(samples)
    t0 = time.perf_counter()
    for (layer, step, pages_l, ctx_t, q_t) in samples:
        ctx = ctx_t.numpy()
        q = q_t.float().double().numpy()
        ts = time.perf_counter()
        for b in range(w.batch):
            n = int(ctx[b])
            n_pages = (n + 15) // 16
            cache = pages_l.index_select(0, tab[b, :n_pages].long()).numpy()
            ident = np.arange(n_pages, dtype=np.int32)[None, :]
            for h in range(Hkv):
                heads = [(0, hq) for hq in range(h * Hg, (h + 1) * Hg)]
                O.decode(cache, ident, [n], q[b:b + 1], st.rot_k[layer], st.rot_v[layer], sm_scale,
                         Hkv, w.group, pairs=heads)
                done_bytes += n * per_tok_head
                pairs += 1
                if time.perf_counter() - ts > share:
                    break
            if time.perf_counter() - ts > share:
                break
    el = time.perf_counter() - t0
    where = ", ".join(f"layer {layer} step {step}" for (layer, step, *_rest) in samples)
    return {"value": round(done_bytes / el / 1e9, 6), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"float64 numpy oracle decode at ({where}), an equal share of "
                      f"{budget_s:.0f} s each: {pairs} (sequence, KV head) pairs x {Hg} query "
                      f"heads in order, BLAS limited to {threads} thread"
                      f"{'s' if threads > 1 else ''}; {el:.1f} s in all"}


def bits_per_element(group: int, head_dim: int = 128) -> float:
    """Stored bits per cached K or V element: 2-bit codes plus one fp16
    (scale, zero) pair per group: 2 + 32 / group."""
    return 2.0 + 32.0 / group


def pages_context(w, ctx0, per_tok_head, prefill):
    """The pages' own figures beside this measurement (none is on MI355X and
    none is a target), and this library's counterparts."""
    import numpy as np
    n = int(np.max(ctx0))
    sink, recent = 64, 256
    body = max(n - sink - recent, 0)
    with_windows = (body * bits_per_element(w.group) + min(n, sink + recent) * 16) / max(n, 1)
    return {
        "pages": [
            {"figure": "decode speed-up vs BF16 FlashDecoding-v2", "value": "up to 3.0x",
             "method": "OScaR", "hardware": "not stated",
             "source": "'The KV cache goes on a diet: INT2 quantization nears lossless', "
                       "'Crush it to INT2'"},
            {"figure": "memory reduction vs BF16", "value": "5.3x", "method": "OScaR",
             "hardware": "not stated", "source": "same page and section"},
            {"figure": "throughput increase vs BF16 FlashDecoding-v2", "value": "4.1x",
             "method": "OScaR", "hardware": "not stated", "source": "same page and section"},
            {"figure": "overhead on decode latency, throughput and prefill time",
             "value": "<= ~2%", "method": "OptR", "hardware": "an NVIDIA GPU",
             "source": "'Pith review of: Output-Aware Rotation for INT2 KV-Cache Quantization', "
                       "'If this is right' and the efficiency figure"},
            {"figure": "effective bits per cache element", "value": 2.32, "method": "OptR",
             "source": "same review, 'The reading' and 'Core claim'"},
        ],
        "this_library": {
            "bits_per_element": bits_per_element(w.group),
            "memory_reduction_vs_bf16": round(16.0 / bits_per_element(w.group), 3),
            "bits_per_element_with_bf16_windows": round(with_windows, 4),
            "windows_context": n,
            "prefill_overhead_pct": (prefill or {}).get("overhead_pct"),
            "note": "bits with windows: the INT2 body plus 64 sink and 256 recent BF16 tokens "
                    "over this context; the overhead compares the encoding kernels only "
                    "(a real prefill adds attention and projections that dilute it)",
        },
    }


def prefill_leg(w, st, table, pages0, mu, rk, rv, dev, reps: int = 3):
    """The prompts of one layer (every sequence's prior context) encoded three
    ways into a scratch cache: with R_K and R_V, with R_V folded into the
    weights (rot_v NULL), and with neither rotation (rot_k and rot_v NULL: the
    plain INT2 cache the rotations are measured against).  Mean of `reps`
    timed calls each, after one warm-up, between HIP events."""
    import numpy as np
    import torch

    import rotated_int2_kv_kvq_amd as kvq
    from workload import kv_for_sequence

    n = int(st.ctx_lens.min())
    if n != int(st.ctx_lens.max()):
        return None  # one call per shared prompt length: the stream workload has one
    kv = [kv_for_sequence(w, st, 0, b, 0, n, dev) for b in range(w.batch)]
    k = torch.stack([x[0] for x in kv]).contiguous()
    v = torch.stack([x[1] for x in kv]).contiguous()
    del kv
    scratch = torch.empty_like(pages0)
    sp = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    modes = {"rotated": (rk, rv), "value_rotation_folded": (rk, None), "unrotated": (None, None)}
    ms = {}
    for name, (a, b_) in modes.items():
        kvq.append(scratch, table, sp, k, v, mu, a, b_, w.group, w.clip_k, w.clip_v)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            kvq.append(scratch, table, sp, k, v, mu, a, b_, w.group, w.clip_k, w.clip_v)
        e1.record()
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / reps
    del k, v, scratch
    tokens = w.batch * n
    base = ms["unrotated"]
    return {
        "call": "kvq_append of the whole prompt, one layer",
        "batch": w.batch, "prompt_tokens": n, "kv_heads": w.num_kv_heads,
        "ms": {k_: round(t, 4) for k_, t in ms.items()},
        "mtok_s": {k_: round(tokens / (t * 1e-3) / 1e6, 3) for k_, t in ms.items()},
        "overhead_pct": {
            "both_rotations_vs_none": round((ms["rotated"] / base - 1) * 100, 2),
            "key_rotation_only_vs_none": round((ms["value_rotation_folded"] / base - 1) * 100, 2),
        },
        "rotation_tflops": round(tokens * w.num_kv_heads * 65536 / (ms["rotated"] * 1e-3) / 1e12, 2),
    }


# Long-context decode workloads, timed cold with the automatic split plan:
# the calls cycle through copies of the cache that together exceed the 256 MB
# Infinity Cache several times, so that each call reads its cache from HBM
# (a flushing write between calls would leave dirty lines whose write-back
# competes with the reads).
LONG_WORKLOADS = ("qwen3_8b_b1_ctx128k_sinks", "qwen3_8b_b64_ctx1k_32k_g64",
                  "qwen3_8b_b4_ctx8k")
COLD_BYTES = 1200 << 20


def build_decode_cache(name: str, dev: str = "cuda"):
    """The INT2 cache of one layer of a workload, built by the bulk append."""
    import numpy as np
    import torch

    import rotated_int2_kv_kvq_amd as kvq
    from workload import WORKLOADS, key_mean, kv_for_sequence, make_static, query_for

    w = WORKLOADS[name]
    st = make_static(w)
    pages = torch.empty(st.num_blocks, w.num_kv_heads, kvq.page_bytes(w.head_dim, w.group),
                        dtype=torch.uint8, device=dev)
    table = torch.from_numpy(st.block_table).to(dev)
    mu = key_mean(w, st, 0, device=dev).contiguous()
    rk = torch.from_numpy(st.rot_k[0]).to(dev).contiguous()
    rv = torch.from_numpy(st.rot_v[0]).to(dev).contiguous()
    chunk = 4096
    for b, n in enumerate(st.ctx_lens):
        for s0 in range(0, int(n), chunk):
            c = min(chunk, int(n) - s0)
            k, v = kv_for_sequence(w, st, 0, b, s0, c, dev)
            kvq.append(pages, table[b:b + 1].contiguous(),
                       torch.full((1,), s0, dtype=torch.int32, device=dev),
                       k[None].contiguous(), v[None].contiguous(), mu, rk, rv, w.group,
                       w.clip_k, w.clip_v)
    q = query_for(w, 0, 0, dev).contiguous()
    ctx = torch.from_numpy(st.ctx_lens.astype(np.int32)).to(dev)
    return w, st, pages, table, ctx, q, rk, rv


def long_context_leg(name: str, reps: int, split_pages: int = 0, cache=None):
    """Cold decode of one layer of a long-context workload: the whole call
    (query rotation, scan, merge) and the scan alone.  Calls run back to back
    over copies of the cache, queued behind a GPU sleep, between one pair of
    events; the figure is the mean per call.  Per-call medians come from an
    event pair around each call: cold (copies cycled) and warm (one copy back
    to back, partly served from the Infinity Cache)."""
    import numpy as np
    import torch

    import rotated_int2_kv_kvq_amd as kvq

    w, st, pages, table, ctx, q, rk, rv = cache or build_decode_cache(name)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    max_ctx = int(st.ctx_lens.max())
    sm = 1.0 / math.sqrt(d)
    nbytes = int(st.ctx_lens.astype(np.int64).sum()) * Hkv * cache_bytes_per_token_head(w.group)
    ncopy = max(2, -(-COLD_BYTES // (pages.numel())))
    copies = [pages] + [pages.clone() for _ in range(ncopy - 1)]
    wsb = kvq.decode_workspace_bytes(B, Hq, Hkv, max_ctx, d, split_pages)
    wss = [torch.empty(wsb, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    calls = max(reps, ncopy)
    # the scan alone: PREPARE and SPLITS together where the plan builds the
    # operand inside the scan (one launch, as in the whole call)
    plan = kvq.decode_plan(B, Hq, Hkv, max_ctx, d, split_pages)
    scan_stages = (kvq.STAGE_PREPARE | kvq.STAGE_SPLITS if plan["operand_in_scan"]
                   else kvq.STAGE_SPLITS)

    def call(i, stages):
        kvq.decode(copies[i % ncopy], table, ctx, max_ctx, q, rk, rv, w.group, sm, out=out,
                   workspace=wss[i % ncopy], split_pages=split_pages, stages=stages)

    full_ms, scan_ms = [], []
    for rep in range(3):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(50_000_000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(calls):
            call(i, kvq.STAGE_ALL)
        e1.record()
        if not plan["operand_in_scan"]:
            for i in range(ncopy):
                call(i, kvq.STAGE_PREPARE)
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(50_000_000)
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e2.record()
        for i in range(calls):
            call(i, scan_stages)
        e3.record()
        torch.cuda.synchronize()
        if rep:
            full_ms.append(e0.elapsed_time(e1) / calls)
            scan_ms.append(e2.elapsed_time(e3) / calls)

    def per_call_us(copy_of):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * calls)]
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(50_000_000)
        for i in range(calls):
            ev[2 * i].record()
            call(copy_of(i), kvq.STAGE_ALL)
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        return float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1])
                                for i in range(1, calls)])) * 1e3

    cold_med = per_call_us(lambda i: i)
    warm_med = per_call_us(lambda i: 0)
    call(0, kvq.STAGE_ALL)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    full_us = float(np.mean(full_ms)) * 1e3
    scan_us = float(np.mean(scan_ms)) * 1e3
    del copies, wss, out
    return {
        "batch": B, "ctx": [int(st.ctx_lens.min()), max_ctx], "group": w.group,
        "cache_bytes": nbytes, "cold": f"{ncopy} cache copies cycled",
        "decode_us": round(full_us, 2),
        "decode_us_median_cold": round(cold_med, 2),
        "decode_us_median_warm": round(warm_med, 2),
        "decode_gbs": round(nbytes / (full_us * 1e-6) / 1e9, 1),
        "decode_frac": round(nbytes / (full_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "scan_us": round(scan_us, 2),
        "scan_gbs": round(nbytes / (scan_us * 1e-6) / 1e9, 1),
        "scan_frac": round(nbytes / (scan_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(B / (full_us * 1e-6), 1),
        "split_pages": split_pages or "auto",
        "splits": plan["num_splits"],
        "scan_kernel": scan_kernel_name(w.group, plan["operand_in_scan"]),
    }


if __name__ == "__main__":
    main()
