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
    return kv + q + o + lse + bt + batch.num_seqs * 8


def source_sha():
    h = hashlib.sha256()
    for f in ("attention.hip", "pa_device.h"):
        with open(os.path.join(ROOT, "attention_paged_kv_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def time_workload(batch, steps, warmup):
    import torch
    from attention_paged_kv_attn_amd import binding as B
    g = batch.to("cuda:0")
    out, lse, ws = B.run_batch(g)            # allocates outputs + workspace once
    torch.cuda.synchronize()
    for _ in range(warmup):
        B.run_batch(g, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    B.paged_attn_kernel_timing_read()         # clear
    B.paged_attn_kernel_timing(True)
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        B.run_batch(g, out=out, lse=lse, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    B.paged_attn_kernel_timing(False)
    a, att, c, n = B.paged_attn_kernel_timing_read()
    ms = t0.elapsed_time(t1) / steps
    return ms, {"assign": a / n, "attention": att / n, "combine": c / n}, (g, out, lse, ws)


def cpu_baseline(batch, budget_s=15.0):
    """The oracle on the first sequences of the batch until ~budget_s of CPU work."""
    from threadpoolctl import threadpool_limits
    from tests.oracle_helpers import run_oracle
    qsl = batch.query_start_loc.numpy()
    done_rows = np.zeros(batch.total_q, bool)
    t_total = 0.0
    nseq = 0
    with threadpool_limits(limits=1):
        for s in range(batch.num_seqs):
            rows = np.zeros(batch.total_q, bool)
            rows[qsl[s]:qsl[s + 1]] = True
            t = time.perf_counter()
            run_oracle(batch, rows=rows)
            t_total += time.perf_counter() - t
            done_rows |= rows
            nseq += 1
            if t_total >= budget_s:
                break
    # algorithmic bytes of the sampled sequences
    ctx = batch.seq_lens.numpy().astype(np.int64)[:nseq]
    d, Hq, Hkv = batch.head_dim, batch.num_q_heads, batch.num_kv_heads
    elt = {"f32": 4, "bf16": 2, "e4m3": 1}[batch.kind]
    nq = int(qsl[nseq])
    by = int(ctx.sum()) * Hkv * d * elt * 2 + nq * Hq * d * (elt + 2) + nq * Hq * 4 + \
        int(((ctx + batch.page_size - 1) // batch.page_size).sum()) * 4
    return {"value": by / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {nseq} of {batch.num_seqs} sequences ({int(ctx.sum())} keys, {nq} query rows) "
                      f"of the same decode batch, fp64 NumPy oracle, BLAS limited to 1 thread, "
                      f"{t_total:.1f} s"}


WORKLOADS = {
    "splitk_decode_q1_NHD": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=1, poison=False),
    "splitk_decode_q2_NHD": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=2, poison=False),
    "splitk_decode_q4_NHD": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=4, poison=False),
    "splitk_decode_q1_HND": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).splitk_decode(q_len=1, kv_layout="HND", poison=False),
    "hybrid_chunked": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).hybrid_chunked(poison=False),
    "prefill_bf16_dense": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sparse_prefill(kind="bf16", mask=False, poison=False),
    "prefill_fp8_tensor_mask": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sparse_prefill(kind="e4m3", quant_mode="tensor", mask=True, poison=False),
    "prefill_fp8_tensor_dense": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sparse_prefill(kind="e4m3", quant_mode="tensor", mask=False, poison=False),
    "window_fwd": lambda: __import__("attention_paged_kv_attn_amd.workloads", fromlist=["x"]).sliding_window(poison=False),
    "window_decode_128k_full": lambda: _full_decode_128k(),
}


def _full_decode_128k():
    from attention_paged_kv_attn_amd import workloads as W
    b = W.sliding_window(decode=True, window=0, landmark_chunk=0, poison=False)
    return b


def leg(name, steps, warmup):
    log(f"generating {name}")
    batch = WORKLOADS[name]()
    pairs, keys = visible_pairs_and_keys(batch)
    by = algorithmic_bytes(batch, keys)
    flops = 4.0 * batch.head_dim * pairs
    log(f"{name}: {by / 1e9:.3f} GB algorithmic, {flops / 1e12:.4f} TFLOP; timing {steps} steps")
    ms, kms, _ = time_workload(batch, steps, warmup)
    log(f"{name}: {ms:.4f} ms/step; kernels {kms}")
    return batch, by, flops, ms, kms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="splitk_decode_q1_NHD", choices=sorted(WORKLOADS))
    ap.add_argument("--prefill-workload", default="prefill_bf16_dense", choices=sorted(WORKLOADS) + ["none"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", default="", help="comma-separated extra workloads to time (reported under 'also')")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

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
        also.append({"workload": name, "ms_per_step": round(ems, 5),
                     "gbs_step": round(eby / (ems * 1e-3) / 1e9, 1),
                     "tflops_attention": round(efl / (ekms["attention"] * 1e-3) / 1e12, 2),
                     "gbs_attention": round(eby / (ekms["attention"] * 1e-3) / 1e9, 1),
                     "kernels_ms": {k: round(v, 5) for k, v in ekms.items()}})
        del eb
    if also:
        result["also"] = also
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(batch)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
