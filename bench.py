#!/usr/bin/env python3
"""Benchmark of the paged-KV attention forward on one MI355X.

A step is one paged_attn_fwd call (Assign -> split-K attention -> Combine)
over one batch whose inputs already sit in HBM.  The headline workload is the
dynamic split-K decode batch with the Llama-3.1-8B attention shape (Hq 32,
Hkv 8, d 128, bf16, 64 sequences with log-uniform contexts 128..32768, 64-token
pages in a random permutation, q_len 1, NHD); its metric is algorithmic HBM
GB/s.  A second leg times the bf16 dense causal prefill at the FP8-prefill
shape (2 x 8192 tokens) for TFLOP/s against the MFMA peak.

Prints ONE JSON line.  Progress goes to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def visible_pairs_and_keys(batch):
    """(sum over rows/heads of visible keys, keys that must be read per kv head)."""
    ctx = batch.seq_lens.cpu().numpy().astype(np.int64)
    qsl = batch.query_start_loc.cpu().numpy().astype(np.int64)
    pairs = 0
    keys = 0
    W, C = batch.window, batch.landmark_chunk
    bm = None if batch.block_mask is None else batch.block_mask.cpu().numpy()
    T = batch.block_mask_tile
    for b in range(len(ctx)):
        ql = int(qsl[b + 1] - qsl[b])
        if ql == 0:
            continue
        pos = ctx[b] - ql + np.arange(ql)
        hi = pos + 1 if batch.causal else np.full(ql, ctx[b])
        lo = np.zeros(ql, dtype=np.int64)
        if W > 0:
            lo = np.maximum(0, pos - W + 1)
            if batch.window_expand_to_chunk and C > 0:
                lo = (lo // C) * C
        if bm is None:
            cnt = hi - lo
            if C > 0:
                cnt = cnt - (hi // C - lo // C)
            pairs += int(cnt.sum())
            need_lo, need_hi = int(lo.min()), int(hi.max())
            k = need_hi - need_lo
            if C > 0:
                k -= need_hi // C - need_lo // C
            keys += k
        else:
            # causal block-sparse prefill: a row in query tile t sees the kept key
            # tiles before t in full and its own tile up to its position
            m = bm[b, 0].astype(bool)
            qt = pos // T
            for t in range(m.shape[0]):
                rows = np.nonzero(qt == t)[0]
                if rows.size == 0:
                    continue
                full_before = int(m[t, :t].sum()) * T
                own = (pos[rows] - t * T + 1) if m[t, t] else np.zeros(rows.size, dtype=np.int64)
                pairs += int((full_before + own).sum())
            kept = (m & np.tril(np.ones_like(m)).astype(bool)).any(axis=0)
            for kt in np.nonzero(kept)[0]:
                keys += int(min(T, ctx[b] - kt * T))
    return pairs * batch.num_q_heads, keys


def algorithmic_bytes(batch, keys_per_head):
    elt = {"f32": 4, "bf16": 2, "e4m3": 1}[batch.kind]
    out_elt = 4 if batch.kind == "f32" else 2
    d, Hq, Hkv = batch.head_dim, batch.num_q_heads, batch.num_kv_heads
    kv = keys_per_head * Hkv * d * elt * 2
    q = batch.total_q * Hq * d * elt
    o = batch.total_q * Hq * d * out_elt
    lse = batch.total_q * Hq * 4
    ctx = batch.seq_lens.cpu().numpy().astype(np.int64)
    bt = int(((ctx + batch.page_size - 1) // batch.page_size).sum()) * 4
    sc = 0
    if batch.scales is not None:                  # fp8 dequantisation scales
        sc = sum(int(batch.scales[w].numel()) * 4 for w in ("q", "k", "v"))
    return kv + q + o + lse + bt + sc + batch.num_seqs * 8


def source_sha():
    h = hashlib.sha256()
    for f in ("attention.hip", "pa_device.h", "combine_core.h"):
        with open(os.path.join(ROOT, "attention_paged_kv_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_summary(workload):
    """The JSON block of profiles/attention_kernel_<workload>.md, or None."""
    path = os.path.join(ROOT, "profiles", f"attention_kernel_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    a = text.find("```json")
    if a < 0:
        return None
    b = text.find("```", a + 7)
    return json.loads(text[a + 7:b])


def traffic_for(workload):
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (scaled by the copy-kernel calibration), if they were taken
    on the current kernel source; else None."""
    t = profile_summary(workload)
    if not t or t.get("source_sha") != source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def split_kw(spec, g):
    """Launch options for a split spec: dynamic, auto (the library's policy,
    decided once on the host before timing) or static<S>."""
    from attention_paged_kv_attn_amd import binding as B
    if spec in (None, "dynamic"):
        return {}
    if spec == "auto":
        params = B.make_params(num_seqs=g.num_seqs, num_q_heads=g.num_q_heads, num_kv_heads=g.num_kv_heads,
                               head_dim=g.head_dim, page_size=g.page_size, num_pages=g.num_pages,
                               max_pages_per_seq=g.block_table.shape[1], total_q=g.total_q,
                               softmax_scale=g.softmax_scale, causal=g.causal, window=g.window,
                               window_expand_to_chunk=g.window_expand_to_chunk, landmark_chunk=g.landmark_chunk)
        mode, S = B.paged_attn_plan_split(params, g.seq_lens, g.query_start_loc, g.block_mask is not None)
        log(f"split policy: {'static S=%d' % S if mode == B.PA_SPLIT_STATIC else 'dynamic'}")
        return {"split": "static", "static_splits": S} if mode == B.PA_SPLIT_STATIC else {}
    if spec.startswith("static"):
        return {"split": "static", "static_splits": int(spec[len("static"):])}
    raise ValueError(spec)


def time_graph(g, kw, steps, warmup):
    """The step captured once in a HIP graph, then replayed: ms per replay."""
    import torch
    from attention_paged_kv_attn_amd import binding as B
    out, lse, ws = B.run_batch(g, **kw)
    for _ in range(warmup):
        B.run_batch(g, out=out, lse=lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.run_batch(g, out=out, lse=lse, workspace=ws, **kw)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_workload(batch, steps, warmup, split=None):
    import torch
    from attention_paged_kv_attn_amd import binding as B
    g = batch.to("cuda:0")
    if split and split.endswith("+graph"):
        kw = split_kw(split[:-len("+graph")] or None, g)
        ms = time_graph(g, kw, steps, warmup)
        return ms, {"assign": float("nan"), "attention": float("nan"), "combine": float("nan")}, None
    kw = split_kw(split, g)
    out, lse, ws = B.run_batch(g, **kw)      # allocates outputs + workspace once
    torch.cuda.synchronize()
    for _ in range(warmup):
        B.run_batch(g, out=out, lse=lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    B.paged_attn_kernel_timing_read()         # clear
    B.paged_attn_kernel_timing(True)
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        B.run_batch(g, out=out, lse=lse, workspace=ws, **kw)
    t1.record(stream)
    torch.cuda.synchronize()
    B.paged_attn_kernel_timing(False)
    a, att, c, n = B.paged_attn_kernel_timing_read()
    ms = t0.elapsed_time(t1) / steps
    return ms, {"assign": a / n, "attention": att / n, "combine": c / n}, (g, out, lse, ws)


def cpu_baseline(batch, budget_s=12.0):
    """The oracle, one sequence at a time in batch order (wrapping round), until
    ~budget_s of CPU work; throughput in the same algorithmic GB/s."""
    from threadpoolctl import threadpool_limits
    from tests.oracle_helpers import run_oracle
    qsl = batch.query_start_loc.numpy().astype(np.int64)
    ctx_all = batch.seq_lens.numpy().astype(np.int64)
    d, Hq, Hkv = batch.head_dim, batch.num_q_heads, batch.num_kv_heads
    elt = {"f32": 4, "bf16": 2, "e4m3": 1}[batch.kind]
    t_total, by, calls, keys = 0.0, 0, 0, 0
    with threadpool_limits(limits=1):
        while t_total < budget_s:
            s = calls % batch.num_seqs
            rows = np.zeros(batch.total_q, bool)
            rows[qsl[s]:qsl[s + 1]] = True
            t = time.perf_counter()
            run_oracle(batch, rows=rows)
            t_total += time.perf_counter() - t
            nq, c = int(qsl[s + 1] - qsl[s]), int(ctx_all[s])
            by += c * Hkv * d * elt * 2 + nq * Hq * d * (elt + 2) + nq * Hq * 4 + \
                (c + batch.page_size - 1) // batch.page_size * 4
            keys += c
            calls += 1
    return {"value": round(by / t_total / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} single-sequence oracle calls over the same decode batch in order "
                      f"({keys} keys, {by / 1e9:.3f} GB algorithmic), fp64 NumPy, BLAS limited to one "
                      f"thread, {t_total:.1f} s"}


WORKLOADS = {
    "splitk_decode_q1_NHD": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=1, poison=False),
    "splitk_decode_q2_NHD": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=2, poison=False),
    "splitk_decode_q4_NHD": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=4, poison=False),
    "splitk_decode_q1_HND": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=1, kv_layout="HND", poison=False),
    "splitk_decode_fp8_q1_NHD": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=1, kind="e4m3", poison=False),
    "splitk_decode_fp8_q2_NHD": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=2, kind="e4m3", poison=False),
    "splitk_decode_fp8_q4_NHD": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=4, kind="e4m3", poison=False),
    "splitk_decode_fp8_q1_HND": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=1, kind="e4m3", kv_layout="HND", poison=False),
    "hybrid_chunked": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).hybrid_chunked(poison=False),
    "prefill_bf16_dense": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sparse_prefill(kind="bf16", mask=False, poison=False),
    "prefill_fp8_tensor_mask": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sparse_prefill(kind="e4m3", quant_mode="tensor", mask=True, poison=False),
    "prefill_fp8_tensor_dense": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sparse_prefill(kind="e4m3", quant_mode="tensor", mask=False, poison=False),
    "window_fwd": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sliding_window(poison=False),
    "window_decode_128k_full": lambda: _full_decode_128k(),
    "window_decode_128k": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sliding_window(decode=True, poison=False),
    "uniform_decode_4k": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).uniform_decode(poison=False),
}


def _full_decode_128k():
    from attention_paged_kv_attn_amd import workloads as W
    b = W.sliding_window(decode=True, window=0, landmark_chunk=0, poison=False)
    return b


def leg(name, steps, warmup):
    """name is a workload, optionally '@dynamic', '@auto' or '@static<S>', and
    '+graph' to time replays of the step captured in a HIP graph."""
    name, _, split = name.partition("@")
    log(f"generating {name}")
    batch = WORKLOADS[name]()
    pairs, keys = visible_pairs_and_keys(batch)
    by = algorithmic_bytes(batch, keys)
    flops = 4.0 * batch.head_dim * pairs
    log(f"{name}: {by / 1e9:.3f} GB algorithmic, {flops / 1e12:.4f} TFLOP; timing {steps} steps")
    ms, kms, _ = time_workload(batch, steps, warmup, split or None)
    log(f"{name}@{split or 'dynamic'}: {ms:.4f} ms/step; kernels {kms}")
    return batch, by, flops, ms, kms


COPY_CALIBRATION_BYTES = 1 << 30


def copy_calibration(launches=5):
    """Plain device-to-device copies of COPY_CALIBRATION_BYTES: the reference
    for scaling FETCH_SIZE / WRITE_SIZE counter readings to bytes."""
    import torch
    src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device="cuda:0")
    src.fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_CALIBRATION_BYTES, "launches": launches}), flush=True)


def _csv_rows(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def _counter_per_dispatch(directory, counter, name_pred):
    vals = [float(r["Counter_Value"]) for r in _csv_rows(directory, "counter_collection.csv")
            if r["Counter_Name"] == counter and name_pred(r["Kernel_Name"])]
    return vals


def summarize_profiles(d):
    """Turn the rocprofv3 CSV output of the profiling commands (listed in
    <d>/commands.txt) into the text summaries under profiles/."""
    cmds = open(os.path.join(d, "commands.txt")).read().strip()
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    is_copy = lambda n: "copy" in n.lower()
    is_att = lambda n: "attention_kernel" in n
    # copy calibration: counter KiB per dispatch against the known byte count
    cf = _counter_per_dispatch(os.path.join(d, "copy_fetch"), "FETCH_SIZE", is_copy)
    cw = _counter_per_dispatch(os.path.join(d, "copy_write"), "WRITE_SIZE", is_copy)
    cf_med, cw_med = float(np.median(cf)), float(np.median(cw))
    f_scale = COPY_CALIBRATION_BYTES / (cf_med * 1024.0)
    w_scale = COPY_CALIBRATION_BYTES / (cw_med * 1024.0)
    with open(os.path.join(out_dir, "copy_calibration.md"), "w") as f:
        f.write("# FETCH_SIZE / WRITE_SIZE calibration on a plain copy kernel\n\n")
        f.write(f"Copy of {COPY_CALIBRATION_BYTES} bytes (1 GiB), {len(cf)} dispatches.\n\n")
        f.write(f"| counter | median KiB per dispatch | bytes it stands for | scale |\n|---|---|---|---|\n")
        f.write(f"| FETCH_SIZE | {cf_med:.1f} | {COPY_CALIBRATION_BYTES} | {f_scale:.4f} |\n")
        f.write(f"| WRITE_SIZE | {cw_med:.1f} | {COPY_CALIBRATION_BYTES} | {w_scale:.4f} |\n\n")
        f.write("Commands:\n\n```\n" + cmds + "\n```\n")
    # full kernel stats of the default bench command
    stats = _csv_rows(os.path.join(d, "trace"), "kernel_stats.csv")
    trace = _csv_rows(os.path.join(d, "trace"), "kernel_trace.csv")
    bench_line = [json.loads(x) for x in open(os.path.join(d, "bench_trace.json")).read().splitlines()
                  if x.startswith("{")][-1]
    att = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
           for r in trace if is_att(r["Kernel_Name"])]
    att.sort()
    steps, warmup = bench_line["steps"], bench_line["warmup"]
    n_dec = 1 + warmup + steps                       # run_batch once, warmup, timed steps
    legs = {bench_line["config"]["workload"]: att[:n_dec]}
    off = n_dec
    events = {bench_line["config"]["workload"]: bench_line["kernels_ms"]["attention"]}
    n_leg = 1 + warmup + max(5, steps // 2)
    if "prefill" in bench_line:
        legs[bench_line["prefill"]["workload"]] = att[off:off + n_leg]
        events[bench_line["prefill"]["workload"]] = bench_line["prefill"]["kernels_ms"]["attention"]
        off += n_leg
    for a in bench_line.get("also", []):
        if "kernels_ms" not in a:                     # a graph replay: launches of its own shape; stop here
            break
        legs[a["workload"]] = att[off:off + n_leg]
        events[a["workload"]] = a["kernels_ms"]["attention"]
        off += n_leg
    with open(os.path.join(out_dir, "bench_default_kernel_stats.md"), "w") as f:
        f.write("# rocprofv3 kernel statistics of the default bench command\n\n")
        f.write("| kernel | calls | average ns | min ns | max ns | % |\n|---|---|---|---|---|---|\n")
        for r in stats:
            f.write(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                    f"{r['MaxNs']} | {r['Percentage']} |\n")
        f.write("\nThe attention kernel serves every leg under one name; the per-dispatch trace splits them "
                "in launch order (first call, warmup, timed steps of each leg):\n\n")
        f.write("| leg | dispatches | average ns (timed steps) | bench HIP-event ms |\n|---|---|---|---|\n")
        for wl, ds in legs.items():
            timed = [x[1] for x in ds[-(steps if wl == bench_line['config']['workload'] else max(5, steps // 2)):]]
            ev = events[wl]
            f.write(f"| {wl} | {len(ds)} | {np.mean(timed):.0f} | {ev} |\n")
        f.write("\nCommands:\n\n```\n" + cmds + "\n```\n")
    # per-workload counter summaries
    for wl in sorted({x[len("fetch_"):] for x in os.listdir(d)
                      if x.startswith("fetch_") and os.path.isdir(os.path.join(d, x))}):
        fv = _counter_per_dispatch(os.path.join(d, f"fetch_{wl}"), "FETCH_SIZE", is_att)
        wv = _counter_per_dispatch(os.path.join(d, f"write_{wl}"), "WRITE_SIZE", is_att)
        fb = float(np.median(fv)) * 1024.0 * f_scale
        wb = float(np.median(wv)) * 1024.0 * w_scale
        timed = None
        if wl in legs:
            k = steps if wl == bench_line["config"]["workload"] else max(5, steps // 2)
            timed = float(np.mean([x[1] for x in legs[wl][-k:]]))
        batch = WORKLOADS[wl]()
        pairs, keys = visible_pairs_and_keys(batch)
        alg = algorithmic_bytes(batch, keys)
        summary = {"workload": wl, "kernel": "attention_kernel", "source_sha": source_sha(),
                   "fetch_kib_median": float(np.median(fv)), "write_kib_median": float(np.median(wv)),
                   "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                   "hbm_bytes_per_launch": int(fb + wb), "algorithmic_bytes": int(alg),
                   "traffic_over_algorithmic": round((fb + wb) / alg, 4),
                   "avg_ns_rocprof": None if timed is None else round(timed),
                   "flops": 4.0 * batch.head_dim * pairs}
        mf = os.path.join(d, f"mfma_{wl}")
        if os.path.isdir(mf):
            rows = _csv_rows(mf, "counter_collection.csv")
            agg = {}
            for r in rows:
                if is_att(r["Kernel_Name"]):
                    agg.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            summary["mfma_counters_median"] = {k: float(np.median(v)) for k, v in agg.items()}
        with open(os.path.join(out_dir, f"attention_kernel_{wl}.md"), "w") as f:
            f.write(f"# attention_kernel on {wl}\n\n")
            f.write(f"HBM traffic per launch: FETCH_SIZE {summary['fetch_kib_median']:.0f} KiB x {f_scale:.3f} + "
                    f"WRITE_SIZE {summary['write_kib_median']:.0f} KiB x {w_scale:.3f} = "
                    f"{summary['hbm_bytes_per_launch'] / 1e6:.1f} MB against {alg / 1e6:.1f} MB algorithmic "
                    f"({summary['traffic_over_algorithmic']:.3f}x).\n\n")
            if timed is not None:
                f.write(f"Average duration of the timed launches in the kernel trace: {timed / 1e3:.1f} us.\n\n")
            mine = "\n".join(c for c in cmds.splitlines()
                             if f" {wl} " in c + " " or "--copy-calibration" in c or "--kernel-trace" in c)
            f.write("```json\n" + json.dumps(summary, indent=1) + "\n```\n\nCommands (the copy runs calibrate "
                    "the counters, the kernel-trace run gives the durations):\n\n```\n" + mine + "\n```\n")
        del batch
    print("wrote summaries to", out_dir)


def profile_leg(name, steps, warmup):
    """One workload only (for counter runs): prints its timing as JSON."""
    batch, by, flops, ms, kms = leg(name, steps, warmup)
    print(json.dumps({"workload": name, "ms_per_step": ms, "kernels_ms": kms}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="splitk_decode_q1_NHD", choices=sorted(WORKLOADS))
    ap.add_argument("--prefill-workload", default="prefill_bf16_dense", choices=sorted(WORKLOADS) + ["none"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", default="splitk_decode_q1_HND,splitk_decode_fp8_q1_NHD",
                    help="comma-separated extra workloads to time (reported under 'also'); '' for none")
    ap.add_argument("--profile-leg", default=None, choices=sorted(WORKLOADS),
                    help="time only this workload (for rocprofv3 counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run plain 1 GiB device copies (counter calibration) and exit")
    ap.add_argument("--summarize-profiles", default=None, metavar="DIR",
                    help="write profiles/*.md from the rocprofv3 CSV output under DIR (CPU only)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    if args.profile_leg:
        profile_leg(args.profile_leg, args.steps, args.warmup)
        return

    batch, by, flops, ms, kms = leg(args.workload, args.steps, args.warmup)
    gbs = by / (ms * 1e-3) / 1e9
    att_gbs = by / (kms["attention"] * 1e-3) / 1e9
    dtype = {"f32": "f32", "bf16": "bf16", "e4m3": "fp8"}[batch.kind]
    result = {
        "metric": "decode HBM GB/s (% peak) + prefill TFLOP/s (% MFMA peak), 8B-shape bf16",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "num_seqs": batch.num_seqs,
                   "num_q_heads": batch.num_q_heads, "num_kv_heads": batch.num_kv_heads,
                   "head_dim": batch.head_dim, "page_size": batch.page_size,
                   "kv_layout": batch.kv_layout, "total_q": batch.total_q,
                   "total_keys": int(batch.seq_lens.sum()), "algorithmic_bytes": by},
        "roofline": {"bound": "hbm", "achieved": round(att_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(att_gbs / HBM_PEAK_GBS, 4), "traffic": traffic_for(args.workload),
                     "kernel": f"attention_kernel<{ {'f32': 0, 'bf16': 1, 'e4m3': 2}[batch.kind] },{batch.head_dim}>"},
        "kernels_ms": {k: round(v, 5) for k, v in kms.items()},
    }
    if args.prefill_workload != "none":
        pb, pby, pfl, pms, pkms = leg(args.prefill_workload, max(5, args.steps // 2), args.warmup)
        peak = FP8_PEAK_TFLOPS if pb.kind == "e4m3" else BF16_PEAK_TFLOPS
        tf = pfl / (pkms["attention"] * 1e-3) / 1e12
        result["prefill"] = {"workload": args.prefill_workload, "ms_per_step": round(pms, 5),
                             "tflops_step": round(pfl / (pms * 1e-3) / 1e12, 2),
                             "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak,
                                          "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                                          "traffic": traffic_for(args.prefill_workload)},
                             "kernels_ms": {k: round(v, 5) for k, v in pkms.items()}}
        del pb
    also = []
    for name in [x for x in args.extra.split(",") if x]:
        eb, eby, efl, ems, ekms = leg(name, max(5, args.steps // 2), args.warmup)
        entry = {"workload": name, "ms_per_step": round(ems, 5), "gbs_step": round(eby / (ems * 1e-3) / 1e9, 1)}
        if ekms["attention"] == ekms["attention"]:          # per-kernel times exist (not a graph replay)
            entry.update({"tflops_attention": round(efl / (ekms["attention"] * 1e-3) / 1e12, 2),
                          "gbs_attention": round(eby / (ekms["attention"] * 1e-3) / 1e9, 1),
                          "kernels_ms": {k: round(v, 5) for k, v in ekms.items()}})
        also.append(entry)
        del eb
    if also:
        result["also"] = also
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(batch)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
