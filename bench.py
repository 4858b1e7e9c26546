#!/usr/bin/env python3
"""Benchmark of the paged-KV attention forward on one MI355X.

A step is one paged_attn_fwd call (Assign -> split-K attention -> Combine)
over one batch whose inputs already sit in HBM.  The headline workload is the
dynamic split-K decode batch with the Llama-3.1-8B attention shape (Hq 32,
Hkv 8, d 128, bf16, 64 sequences with log-uniform contexts 128..32768, 64-token
pages in a random permutation, q_len 1, NHD); its metric is algorithmic HBM
GB/s, and the same step is also timed replayed from a HIP graph.  The
`prefill` leg times the bf16 dense causal prefill at the FP8-prefill shape
(2 x 8192 tokens) for TFLOP/s against the MFMA peak.  The `also` legs cover
the other workloads: the decode batch in HND, at q_len 2 and 4 and in fp8;
the hybrid chunked step; FP8 prefill dense and block-sparse (tile-skip ratio,
speed-up over its dense run); the sliding-window forward; the windowed and
full 128K decodes under the split policy.  Every leg carries a roofline
object for its attention kernel (HBM or MFMA bound); legs whose working set
is under 1 GB read a 1 GiB buffer between timed steps so their data comes
from HBM.  A streaming-bandwidth figure of torch's own kernels and the fp64
oracle timed on the host's cores (decode batch and sampled prefill rows)
give context.

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


# attention-kernel launches per leg, in execution order (the kernel-trace
# summary slices the trace by these counts)
LAUNCH_LOG = []
_FLUSH = None
FLUSH_BYTES = 1 << 30
FLUSH_BELOW_BYTES = 1_000_000_000


# Warm-up: the W untimed steps, then more until the leg's step has run
# back to back for this long.  A leg starts after seconds of host-side input
# generation with the GPU idle; its first ~50 ms of steps measured 5-15%
# slower on MI355X (prefill 1.04-1.09 ms against 0.98-1.00 ms once warm).
MIN_WARMUP_S = 0.25


def warm_up(run, warmup):
    """Runs `run` warmup times, then in batches of 8 until MIN_WARMUP_S of
    wall time has passed; returns the number of calls."""
    import torch
    n = 0
    for _ in range(warmup):
        run()
        n += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < MIN_WARMUP_S:
        for _ in range(8):
            run()
        n += 8
        torch.cuda.synchronize()
    return n


def flush_caches():
    """Read a 1 GiB scratch buffer: evicts the L2s and the 256 MiB MALL with
    clean lines, so a working set under 1 GB is read from HBM on every timed
    step.  (Writing the buffer instead leaves up to the MALL's size in dirty
    lines, whose write-back then runs inside the next timed kernel: measured
    0.156 -> 0.219 ms on the 0.7 GB fp8 decode batch.)"""
    import torch
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    _FLUSH.sum()


def time_graph(g, kw, steps, warmup, leg_name):
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
    n_warm = warm_up(graph.replay, warmup)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    LAUNCH_LOG.append((leg_name, 1 + warmup + n_warm + steps, steps))
    return t0.elapsed_time(t1) / steps


def time_workload(batch, steps, warmup, split=None, flush=False, leg_name=None, g=None):
    """Eager steps: returns (ms per step, per-kernel ms, flushed).  With
    `flush`, a 1 GiB read runs before every timed step, outside its events.

    The steps are timed twice: first as they run in use, then with the
    library's per-kernel event records on (paged_attn_kernel_timing), which
    give the per-kernel times.  Those records add packets between the three
    launches of a step (measured +13 us on the 0.25 ms decode step), so the
    step time comes from the first pass and the per-kernel times from the
    second, the last `steps` launches of the leg."""
    import torch
    from attention_paged_kv_attn_amd import binding as B
    g = batch.to("cuda:0") if g is None else g
    leg_name = leg_name or batch.name
    if split and split.endswith("+graph"):
        kw = split_kw(split[:-len("+graph")] or None, g)
        ms = time_graph(g, kw, steps, warmup, leg_name)
        return ms, {"assign": float("nan"), "attention": float("nan"), "combine": float("nan")}, False
    kw = split_kw(split, g)
    out, lse, ws = B.run_batch(g, **kw)      # allocates outputs + workspace once
    torch.cuda.synchronize()
    n_warm = warm_up(lambda: B.run_batch(g, out=out, lse=lse, workspace=ws, **kw), warmup)
    stream = torch.cuda.current_stream()

    def timed_pass(instrumented):
        if instrumented:
            B.paged_attn_kernel_timing_read()         # clear
            B.paged_attn_kernel_timing(True)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        if not flush:
            ev[0][0].record(stream)
        for i in range(steps):
            if flush:
                flush_caches()
                ev[i][0].record(stream)
            B.run_batch(g, out=out, lse=lse, workspace=ws, **kw)
            if flush:
                ev[i][1].record(stream)
        if not flush:
            ev[-1][1].record(stream)
        torch.cuda.synchronize()
        if flush:
            ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps
        else:
            ms = ev[0][0].elapsed_time(ev[-1][1]) / steps
        if not instrumented:
            return ms, None
        B.paged_attn_kernel_timing(False)
        a, att, c, n = B.paged_attn_kernel_timing_read()
        return ms, {"assign": a / n, "attention": att / n, "combine": c / n}

    ms, _ = timed_pass(False)
    _, kms = timed_pass(True)
    LAUNCH_LOG.append((leg_name, 1 + n_warm + 2 * steps, steps))
    return ms, kms, flush


def _cpu_threads():
    """Threads the CPU baseline may use: the machine's CPU share when the launcher
    states it (OMP_NUM_THREADS), else every core."""
    return int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)


def _blas_threads():
    from threadpoolctl import threadpool_info
    return max((int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"),
               default=1)


def cpu_baseline(batch, by, budget_s=10.0):
    """The oracle over the whole headline batch, repeated until ~budget_s of
    CPU work, on the host's cores; algorithmic GB/s as the GPU figure."""
    from threadpoolctl import threadpool_limits
    from tests.oracle_helpers import run_oracle
    n = _cpu_threads()
    t_total, calls = 0.0, 0
    with threadpool_limits(limits=n):
        blas = _blas_threads()
        while t_total < budget_s:
            t = time.perf_counter()
            run_oracle(batch)
            t_total += time.perf_counter() - t
            calls += 1
    return {"value": round(by * calls / t_total / 1e9, 3), "unit": "GB/s", "cores": blas, "kind": "oracle",
            "os_cpu_count": os.cpu_count(), "blas_threads": blas,
            "sample": f"{calls} oracle passes over the whole {batch.name} batch ({batch.num_seqs} sequences, "
                      f"{int(batch.seq_lens.sum())} keys, {by / 1e9:.3f} GB algorithmic each), fp64 NumPy, "
                      f"BLAS on {blas} threads, {t_total:.1f} s"}


def cpu_baseline_prefill(batch, budget_s=10.0, rows_per_seq=32):
    """The oracle on sampled query rows of the prefill batch (evenly spaced
    positions, every head), until ~budget_s; TFLOP/s of the visible work."""
    from threadpoolctl import threadpool_limits
    from tests.oracle_helpers import run_oracle
    qsl = batch.query_start_loc.numpy().astype(np.int64)
    rows = np.zeros(batch.total_q, bool)
    for b in range(batch.num_seqs):
        ql = int(qsl[b + 1] - qsl[b])
        rows[qsl[b] + np.unique(np.linspace(0, ql - 1, rows_per_seq).astype(np.int64))] = True
    sub_pairs = 0
    ctx = batch.seq_lens.numpy().astype(np.int64)
    for b in range(batch.num_seqs):
        r = np.nonzero(rows[qsl[b]:qsl[b + 1]])[0]
        sub_pairs += int((ctx[b] - (qsl[b + 1] - qsl[b]) + r + 1).sum())   # causal, no mask
    flops = 4.0 * batch.head_dim * batch.num_q_heads * sub_pairs
    n = _cpu_threads()
    t_total, calls = 0.0, 0
    with threadpool_limits(limits=n):
        blas = _blas_threads()
        while t_total < budget_s:
            t = time.perf_counter()
            run_oracle(batch, rows=rows)
            t_total += time.perf_counter() - t
            calls += 1
    return {"value": round(flops * calls / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": blas,
            "kind": "oracle", "sample": f"{calls} oracle passes over {int(rows.sum())} query rows x "
                                        f"{batch.num_q_heads} heads of {batch.name} (evenly spaced positions), "
                                        f"{flops / 1e9:.1f} GFLOP each, BLAS on {blas} threads, {t_total:.1f} s"}


def stream_bandwidth():
    """Context only: torch's own streaming kernels on 2 GiB (a sum reads it,
    a copy reads and writes it); GB/s of bytes moved."""
    import torch
    n = 1 << 29
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    res = {}
    for name, fn, moved in (("read_sum", lambda: x.sum(), 4 * n), ("copy", lambda: y.copy_(x), 8 * n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(10):
            fn()
        t1.record()
        torch.cuda.synchronize()
        res[name] = round(moved * 10 / (t0.elapsed_time(t1) * 1e-3) / 1e9, 1)
    del x, y
    return {"unit": "GB/s", **res, "kernels": "torch sum / copy_ over 2 GiB fp32 (context, not a target)"}


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
    "prefill_fp8_page_head_mask": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sparse_prefill(kind="e4m3", quant_mode="page_head", mask=True, poison=False),
    "prefill_fp8_page_head_dense": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sparse_prefill(kind="e4m3", quant_mode="page_head", mask=False, poison=False),
    "window_fwd": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sliding_window(poison=False),
    "window_decode_128k_full": lambda: _full_decode_128k(),
    "window_decode_128k": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sliding_window(decode=True, poison=False),
    "uniform_decode_4k": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).uniform_decode(poison=False),
}


def _full_decode_128k():
    from attention_paged_kv_attn_amd import workloads as W
    b = W.sliding_window(decode=True, window=0, landmark_chunk=0, poison=False)
    return b


# how each workload is bounded: HBM bytes (decode-like) or MFMA flops (prefill-like)
MFMA_BOUND = {"prefill_bf16_dense", "prefill_fp8_tensor_dense", "prefill_fp8_tensor_mask",
              "prefill_fp8_page_head_dense", "prefill_fp8_page_head_mask", "window_fwd"}

# the default run: every config's timing leg after the headline decode and the
# bf16 dense prefill (C2 MTP and layouts, C2 fp8, C3, C4 fp8, C5 and its decodes)
DEFAULT_EXTRA = ("splitk_decode_q1_HND,splitk_decode_q2_NHD,splitk_decode_q4_NHD,splitk_decode_fp8_q1_NHD,"
                 "hybrid_chunked,prefill_fp8_tensor_dense,prefill_fp8_tensor_mask,window_fwd,"
                 "window_decode_128k@auto,window_decode_128k_full@auto")


def roofline_of(name, batch, by, flops, att_ms):
    """The roofline object of one leg's attention kernel: algorithmic work per
    launch over its mean launch time (HIP events on the kernel's stream)."""
    wl = name.partition("@")[0]
    if wl in MFMA_BOUND:
        peak = FP8_PEAK_TFLOPS if batch.kind == "e4m3" else BF16_PEAK_TFLOPS
        ach = flops / (att_ms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
             "frac": round(ach / peak, 4)}
    else:
        ach = by / (att_ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4)}
    r["traffic"] = traffic_for(wl)
    prof = profile_summary(wl)
    if prof and prof.get("source_sha") == source_sha() and prof.get("mfma_busy") is not None:
        r["mfma_busy"] = prof["mfma_busy"]              # rocprof: MFMA busy / (SIMDs x active cycles)
        r["clock_ghz"] = prof.get("clock_ghz")
    return r


def leg(name, steps, warmup):
    """name is a workload, optionally '@dynamic', '@auto' or '@static<S>', and
    '+graph' to time replays of the step captured in a HIP graph."""
    wl, _, split = name.partition("@")
    log(f"generating {wl}")
    batch = WORKLOADS[wl]()
    pairs, keys = visible_pairs_and_keys(batch)
    by = algorithmic_bytes(batch, keys)
    flops = 4.0 * batch.head_dim * pairs
    flush = by < FLUSH_BELOW_BYTES and not split.endswith("+graph")
    log(f"{name}: {by / 1e9:.3f} GB algorithmic, {flops / 1e12:.4f} TFLOP; timing {steps} steps"
        f"{' (caches flushed between steps)' if flush else ''}")
    ms, kms, flushed = time_workload(batch, steps, warmup, split or None, flush=flush, leg_name=name)
    log(f"{name}: {ms:.4f} ms/step; kernels {kms}")
    return batch, by, flops, ms, kms, flushed


def leg_entry(name, batch, by, flops, ms, kms, flushed):
    e = {"workload": name, "ms_per_step": round(ms, 5), "flushed": flushed,
         "algorithmic_bytes": int(by), "flops": flops}
    if kms["attention"] == kms["attention"]:            # per-kernel times exist (not a graph replay)
        e["kernels_ms"] = {k: round(v, 5) for k, v in kms.items()}
        e["roofline"] = roofline_of(name, batch, by, flops, kms["attention"])
        e["gbs_attention"] = round(by / (kms["attention"] * 1e-3) / 1e9, 1)
        e["tflops_attention"] = round(flops / (kms["attention"] * 1e-3) / 1e12, 2)
    if "tile_skip_ratio" in batch.info:
        e["tile_skip_ratio"] = round(batch.info["tile_skip_ratio"], 4)
    return e


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


N_XCD, N_CU, N_SIMD = 8, 256, 1024        # MI355X: counters summed over XCDs, SIMDs per device


def derive_counters(c, avg_ns):
    """Utilisations from raw counter sums of one dispatch, by rocprof's own
    formulas for gfx950 (GRBM_GUI_ACTIVE summed over the 8 XCDs is 8x the
    per-XCD active cycles)."""
    out = {}
    gui = c.get("GRBM_GUI_ACTIVE")
    if not gui:
        return out
    cyc = gui / N_XCD
    out["active_cycles"] = round(cyc)
    if avg_ns:
        out["clock_ghz"] = round(cyc / avg_ns, 3)
    if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out["mfma_busy"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc), 4)
    for k in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8"):
        if k in c:
            out["mfma_flops_" + k.rsplit("_", 1)[1].lower()] = c[k] * 512
    if "SQ_ACTIVE_INST_VALU" in c:
        out["valu_active"] = round(c["SQ_ACTIVE_INST_VALU"] / (N_CU * cyc), 4)
    if "SQ_LDS_IDX_ACTIVE" in c:
        out["lds_idx_active"] = round(c["SQ_LDS_IDX_ACTIVE"] / (N_CU * cyc), 4)
        if "SQ_LDS_BANK_CONFLICT" in c:
            out["lds_bank_conflict_ratio"] = round(c["SQ_LDS_BANK_CONFLICT"] /
                                                   max(1.0, c["SQ_LDS_IDX_ACTIVE"] - c["SQ_LDS_BANK_CONFLICT"]), 4)
    return out


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
        f.write("| counter | median KiB per dispatch | bytes it stands for | scale |\n|---|---|---|---|\n")
        f.write(f"| FETCH_SIZE | {cf_med:.1f} | {COPY_CALIBRATION_BYTES} | {f_scale:.4f} |\n")
        f.write(f"| WRITE_SIZE | {cw_med:.1f} | {COPY_CALIBRATION_BYTES} | {w_scale:.4f} |\n\n")
        f.write("Commands:\n\n```\n" + "\n".join(c for c in cmds.splitlines() if "copy" in c) + "\n```\n")
    # the kernel trace of the default bench command, split by its launch log
    stats = _csv_rows(os.path.join(d, "trace"), "kernel_stats.csv")
    trace = _csv_rows(os.path.join(d, "trace"), "kernel_trace.csv")
    bench_line = [json.loads(x) for x in open(os.path.join(d, "bench_trace.json")).read().splitlines()
                  if x.startswith("{")][-1]
    att = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                 for r in trace if is_att(r["Kernel_Name"]))
    events = {bench_line["config"]["workload"]: bench_line["kernels_ms"]["attention"]}
    for e in ([bench_line["prefill"]] if "prefill" in bench_line else []) + bench_line.get("also", []):
        if "kernels_ms" in e:
            events[e["workload"]] = e["kernels_ms"]["attention"]
    legs, off = {}, 0
    for name, total, timed in bench_line["launch_log"]:
        ds = att[off:off + total]
        off += total
        legs[name] = (len(ds), float(np.mean([x[1] for x in ds[-timed:]])) if ds else float("nan"))
    assert off == len(att), f"launch log covers {off} of {len(att)} attention dispatches"
    with open(os.path.join(out_dir, "bench_default_kernel_stats.md"), "w") as f:
        f.write("# rocprofv3 kernel statistics of the default bench command\n\n")
        f.write("| kernel | calls | average ns | min ns | max ns | % |\n|---|---|---|---|---|---|\n")
        for r in stats:
            f.write(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                    f"{r['MaxNs']} | {r['Percentage']} |\n")
        f.write("\nThe attention kernel serves every leg under one name; the per-dispatch trace is split by the "
                "bench's launch log (first call, warmup and timed steps of each leg, in order; a graph leg "
                "also counts its eager warmup):\n\n")
        f.write("| leg | dispatches | average ns (timed steps) | bench HIP-event ms |\n|---|---|---|---|\n")
        for name, (n, avg) in legs.items():
            f.write(f"| {name} | {n} | {avg:.0f} | {events.get(name, '(graph replay)')} |\n")
        f.write("\nCommand:\n\n```\n" + "\n".join(c for c in cmds.splitlines() if "--kernel-trace" in c) +
                "\n```\n")
    # per-workload counter summaries
    for wl in sorted({x[len("fetch_"):] for x in os.listdir(d)
                      if x.startswith("fetch_") and os.path.isdir(os.path.join(d, x))}):
        fv = _counter_per_dispatch(os.path.join(d, f"fetch_{wl}"), "FETCH_SIZE", is_att)
        wv = _counter_per_dispatch(os.path.join(d, f"write_{wl}"), "WRITE_SIZE", is_att)
        fb = float(np.median(fv)) * 1024.0 * f_scale
        wb = float(np.median(wv)) * 1024.0 * w_scale
        timed = next((avg for name, (n, avg) in legs.items() if name.partition("@")[0] == wl), None)
        batch = WORKLOADS[wl]()
        pairs, keys = visible_pairs_and_keys(batch)
        alg = algorithmic_bytes(batch, keys)
        flops = 4.0 * batch.head_dim * pairs
        summary = {"workload": wl, "kernel": "attention_kernel", "source_sha": source_sha(),
                   "fetch_kib_median": float(np.median(fv)), "write_kib_median": float(np.median(wv)),
                   "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                   "hbm_bytes_per_launch": int(fb + wb), "algorithmic_bytes": int(alg),
                   "traffic_over_algorithmic": round((fb + wb) / alg, 4),
                   "avg_ns_rocprof": None if timed is None else round(timed), "flops": flops}
        counters = {}
        for pas in ("mfma", "pipe"):
            pd = os.path.join(d, f"{pas}_{wl}")
            if os.path.isdir(pd):
                agg = {}
                for r in _csv_rows(pd, "counter_collection.csv"):
                    if is_att(r["Kernel_Name"]):
                        agg.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                med = {k: float(np.median(v)) for k, v in agg.items()}
                summary[f"{pas}_counters_median"] = med
                # GRBM_GUI_ACTIVE of each pass goes with that pass's counters
                counters.update({k: v for k, v in med.items() if k != "GRBM_GUI_ACTIVE" or pas == "mfma"})
        derived = derive_counters(counters, timed)
        summary.update(derived)
        peak = FP8_PEAK_TFLOPS if batch.kind == "e4m3" else BF16_PEAK_TFLOPS
        with open(os.path.join(out_dir, f"attention_kernel_{wl}.md"), "w") as f:
            f.write(f"# attention_kernel on {wl}\n\n")
            f.write(f"HBM traffic per launch: FETCH_SIZE {summary['fetch_kib_median']:.0f} KiB x {f_scale:.3f} + "
                    f"WRITE_SIZE {summary['write_kib_median']:.0f} KiB x {w_scale:.3f} = "
                    f"{summary['hbm_bytes_per_launch'] / 1e6:.1f} MB against {alg / 1e6:.1f} MB algorithmic "
                    f"({summary['traffic_over_algorithmic']:.3f}x).\n\n")
            if timed is not None:
                f.write(f"Average duration of the timed launches in the kernel trace: {timed / 1e3:.1f} us "
                        f"({alg / timed:.0f} GB/s algorithmic, {flops / timed / 1e3:.1f} TFLOP/s = "
                        f"{flops / timed / 1e3 / peak:.3f} of the {peak:.0f} TFLOP/s "
                        f"{'fp8' if batch.kind == 'e4m3' else 'bf16'} peak).\n\n")
            if "mfma_busy" in derived:
                f.write(f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({N_SIMD} SIMDs x active cycles) = "
                        f"**{derived['mfma_busy']:.3f}**; active cycles = GRBM_GUI_ACTIVE / {N_XCD} XCDs = "
                        f"{derived['active_cycles']}, so the clock during the kernel was "
                        f"{derived.get('clock_ghz')} GHz.\n\n")
            if "valu_active" in derived:
                f.write(f"VALU active (SQ_ACTIVE_INST_VALU / ({N_CU} CUs x active cycles), rocprof's VALU "
                        f"utilisation formula) = {derived['valu_active']:.3f}; LDS active (SQ_LDS_IDX_ACTIVE / "
                        f"(CUs x cycles)) = {derived.get('lds_idx_active')}; bank conflicts per conflict-free "
                        f"LDS cycle = {derived.get('lds_bank_conflict_ratio')}.\n\n")
            mine = "\n".join(c for c in cmds.splitlines()
                             if f" {wl} " in c + " " or "--copy-calibration" in c or "--kernel-trace" in c)
            f.write("```json\n" + json.dumps(summary, indent=1) + "\n```\n\nCommands (the copy runs calibrate "
                    "the counters, the kernel-trace run gives the durations):\n\n```\n" + mine + "\n```\n")
        del batch
    print("wrote summaries to", out_dir)


def profile_leg(name, steps, warmup):
    """One workload only (for counter runs, which count every dispatch: the
    timed-warm-up is off so that the W warm-up steps and the timed ones are
    all there is): prints its timing as JSON."""
    global MIN_WARMUP_S
    MIN_WARMUP_S = 0.0
    batch, by, flops, ms, kms, flushed = leg(name, steps, warmup)
    print(json.dumps({"workload": name, "ms_per_step": ms, "kernels_ms": kms}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed steps per leg (then more, back to back, until MIN_WARMUP_S has passed)")
    ap.add_argument("--workload", default="splitk_decode_q1_NHD", choices=sorted(WORKLOADS))
    ap.add_argument("--prefill-workload", default="prefill_bf16_dense", choices=sorted(WORKLOADS) + ["none"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the headline step")
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
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

    # the flush buffer is allocated and read once before any leg: the steps
    # that followed its first allocation measured 8-15% slower for tens of
    # milliseconds (bf16 prefill 1.05-1.14 ms against 0.98 ms), which landed
    # on the first flushed leg
    flush_caches()
    torch.cuda.synchronize()
    batch, by, flops, ms, kms, flushed = leg(args.workload, args.steps, args.warmup)
    gbs = by / (ms * 1e-3) / 1e9
    dtype = {"f32": "f32", "bf16": "bf16", "e4m3": "fp8"}[batch.kind]
    roof = roofline_of(args.workload, batch, by, flops, kms["attention"])
    roof["kernel"] = f"attention_kernel<{ {'f32': 0, 'bf16': 1, 'e4m3': 2}[batch.kind] },{batch.head_dim}>"
    result = {
        "metric": "decode HBM GB/s (% peak) + prefill TFLOP/s (% MFMA peak), 8B-shape bf16",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_note": f"per leg: {args.warmup} steps, then back to back until {MIN_WARMUP_S} s",
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
        "roofline": roof,
        "kernels_ms": {k: round(v, 5) for k, v in kms.items()},
        "timing_note": "ms_per_step from steps as run in use; kernels_ms (and roofline.achieved) from a "
                       "second pass with the library's per-kernel event records on",
        "flushed": flushed,
    }
    if not args.no_graph:
        gms, _, _ = time_workload(batch, args.steps, args.warmup, split="dynamic+graph",
                                  leg_name=args.workload + "+graph")
        result["graph_replay"] = {"ms_per_step": round(gms, 5), "gbs_step": round(by / (gms * 1e-3) / 1e9, 1)}
        log(f"{args.workload} replayed from a HIP graph: {gms:.4f} ms/step")
    head_batch, head_by = batch, by
    legs = {}
    if args.prefill_workload != "none":
        r = leg(args.prefill_workload, max(5, args.steps // 2), args.warmup)
        pb, pfl, pms = r[0], r[2], r[3]
        e = leg_entry(args.prefill_workload, *r)
        e["tflops_step"] = round(pfl / (pms * 1e-3) / 1e12, 2)
        result["prefill"] = e
        legs[args.prefill_workload] = e
        del pb
    also = []
    for name in [x for x in args.extra.split(",") if x]:
        r = leg(name, max(5, args.steps // 2), args.warmup)
        e = leg_entry(name, *r)
        also.append(e)
        legs[name] = e
        del r
    # block-sparse prefill against its own dense run (same quantisation)
    for m in [x for x in legs if x.endswith("_mask")]:
        dense = m[:-len("_mask")] + "_dense"
        if dense in legs and "kernels_ms" in legs[m] and "kernels_ms" in legs[dense]:
            legs[m]["speedup_vs_dense"] = round(legs[dense]["kernels_ms"]["attention"] /
                                                legs[m]["kernels_ms"]["attention"], 3)
    if also:
        result["also"] = also
    result["stream_bandwidth"] = stream_bandwidth()
    result["launch_log"] = LAUNCH_LOG
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(head_batch, head_by)
        if args.prefill_workload != "none":
            result["cpu_baseline"]["prefill"] = cpu_baseline_prefill(WORKLOADS[args.prefill_workload]())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
