"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances (max abs error over every compared element):
  bf16 inputs  O <= 2e-2, LSE <= 1e-3   (fp32 accumulation, P rounded to bf16)
  fp8  inputs  O <= 4e-2, LSE <= 1e-3   (against the oracle on dequantised inputs)
  fp32 inputs  O <= 1e-5, LSE <= 1e-5
Task-map and index work: bit-exact.  The decode and hybrid workloads are
compared at full size on every row; the 2 x 8192 prefill and the 8192-token
sliding-window forward at full size on sampled query rows that the oracle
computes one by one.  Each comparison also logs the relative RMS error of O.
"""
import math
import sys

import numpy as np
import pytest
import torch

from attention_paged_kv_attn_amd import binding as B
from attention_paged_kv_attn_amd import workloads as W
from oracle import taskmap
from tests import parity_log
from tests.oracle_helpers import run_oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-3), "e4m3": (4e-2, 1e-3), "f32": (1e-5, 1e-5)}
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_run(batch, **kw):
    g = batch.to(DEV)
    say(f"  launch {batch.name} total_q={batch.total_q} B={batch.num_seqs} kw={kw}")
    out, lse, ws = B.run_batch(g, **kw)
    torch.cuda.synchronize()
    return g, out, lse, ws


def header(ws, params):
    lay = B.paged_attn_workspace_layout(params)
    h = ws[lay.header:lay.header + 64].cpu().view(torch.int32).numpy()
    return h, lay


def params_of(g, **kw):
    args = dict(num_seqs=g.num_seqs, num_q_heads=g.num_q_heads, num_kv_heads=g.num_kv_heads,
                head_dim=g.head_dim, page_size=g.page_size, num_pages=g.num_pages,
                max_pages_per_seq=g.block_table.shape[1], total_q=g.total_q,
                softmax_scale=g.softmax_scale, causal=g.causal, window=g.window,
                window_expand_to_chunk=g.window_expand_to_chunk, landmark_chunk=g.landmark_chunk,
                block_mask_tile=g.block_mask_tile)
    args.update(kw)
    return B.make_params(**args)


def compare(batch, out, lse, rows=None, tol=None, **oracle_kw):
    O, L = run_oracle(batch, rows=rows, **oracle_kw)
    o = out.float().cpu().numpy()
    l = lse.float().cpu().numpy()
    sel = np.ones(batch.total_q, bool) if rows is None else np.asarray(rows)
    to, tl = tol or TOL[batch.kind]
    assert np.all(np.isfinite(o[sel])), "non-finite output"
    d = o[sel] - O[sel]
    eo = np.abs(d).max()
    # relative RMS error of O: small outputs at long context make max-abs alone
    # a weak measure (|O| ~ 0.02-0.1 there)
    rel_rms = float(np.sqrt(np.mean(d * d) / max(np.mean(O[sel] * O[sel]), 1e-300)))
    # rows with no visible key: LSE -inf on both sides counts as equal, and
    # -inf on one side only fails
    ls, Ls = l[sel], L[sel]
    both = np.isneginf(ls) & np.isneginf(Ls)
    assert np.array_equal(np.isneginf(ls), np.isneginf(Ls)), "rows without visible keys differ"
    el = float(np.abs(ls[~both] - Ls[~both]).max()) if (~both).any() else 0.0
    say(f"  {batch.name}: max|dO|={eo:.3e} relRMS(O)={rel_rms:.3e} max|dLSE|={el:.3e} rows={int(sel.sum())}")
    parity_log.record(None, batch.name, batch.kind, int(sel.sum()), eo, rel_rms, el)
    assert eo <= to, f"O error {eo} > {to}"
    assert el <= tl, f"LSE error {el} > {tl}"
    return eo, el


def check_no_device_error(ws, g, **kw):
    h, _ = header(ws, params_of(g, **kw))
    assert h[7] == 0, f"device error word {h[7]}"
    return h


def effective_pair_weight(b, weight=0):
    """The library's pair weight for a run_batch call (which states the batch's max_q_len)."""
    if weight:
        return weight
    small = b.max_q_len * (b.num_q_heads // b.num_kv_heads) <= 16
    return B.PA_PAIR_WEIGHT_SMALL if small else B.PA_PAIR_WEIGHT_GENERAL


def sequence_qblocks(b, **kw):
    """Whether the library cuts a run_batch call on b into one Q-block per
    sequence (the layout reports the query heads per Q-block)."""
    if b.block_mask is not None:
        return False
    lay = B.paged_attn_workspace_layout(params_of(b, max_q_len=kw.get("max_q_len", b.max_q_len),
                                                  qblock_per_kv_head=int(kw.get("qblock_per_kv_head", 0))))
    return lay.qblock_heads != b.num_q_heads // b.num_kv_heads


def oracle_taskmap(b, P, force=0, weight=0, **kw):
    return taskmap.build(b.seq_lens.numpy(), b.query_start_loc.numpy(), Hq=b.num_q_heads,
                         Hkv=b.num_kv_heads, num_workers=P, split_min_units=8, force_split_units=force,
                         pair_weight=effective_pair_weight(b, weight),
                         causal=b.causal, window=b.window, window_expand_to_chunk=b.window_expand_to_chunk,
                         landmark_chunk=b.landmark_chunk,
                         block_mask=None if b.block_mask is None else b.block_mask.numpy(),
                         block_mask_tile=b.block_mask_tile, heads_interleaved=sequence_qblocks(b, **kw))


def slots_for(b, P, force, weight=0, **kw):
    """Partial slots a forced split needs (the default 2 P covers natural splits)."""
    return max(1, oracle_taskmap(b, P, force, weight, **kw)["n_slots"]) if force else 0


def sample_rows(total_q, k, seed=0, must=()):
    rng = np.random.default_rng(seed)
    m = np.zeros(total_q, bool)
    m[rng.choice(total_q, size=min(k, total_q), replace=False)] = True
    m[list(must)] = True
    return m


# ---------------------------------------------------------------------------
def test_device_info():
    info = B.paged_attn_device_info(0)
    say(f"  device {info}")
    assert info["compute_units"] > 0 and "gfx950" in info["arch"]


@pytest.mark.parametrize("make", [
    lambda: W.tiny_hybrid(),
    lambda: W.splitk_decode(q_len=1, batch=16, ctx_lo=64, ctx_hi=3000),
    lambda: W.splitk_decode(q_len=[1, 2, 4, 3] * 4, batch=16, ctx_lo=64, ctx_hi=3000),
    lambda: W.hybrid_chunked(batch=12, chunk=200, history=700, dec_lo=100, dec_hi=2000),
    lambda: W.sparse_prefill(kind="bf16", seq_len=1024),
    lambda: W.sparse_prefill(kind="bf16", seq_len=1000, mask=False),
    lambda: W.sparse_prefill(kind="e4m3", seq_len=1000, mask=False),
    lambda: W.sliding_window(seq_len=1500, window=512),
], ids=["tiny", "decode", "mtp_mix", "hybrid", "sparse", "dense_lean", "dense_lean_fp8", "window"])
@pytest.mark.parametrize("workers,force,weight", [(0, 0, 0), (0, 0, 73), (7, 0, 0), (64, 0, 35), (37, 1, 0),
                                                  (5, 3, 90)])
def test_taskmap_bit_exact(make, workers, force, weight):
    b = make()
    info = B.paged_attn_device_info(0)
    P = workers or info["default_workers"]
    ref = oracle_taskmap(b, P, force, weight)
    slots = slots_for(b, P, force, weight)
    g, out, lse, ws = gpu_run(b, num_workers=workers, force_split_units=force, max_partial_slots=slots,
                              pair_weight=weight)
    params = params_of(g, num_workers=workers, force_split_units=force, max_partial_slots=slots)
    h, lay = header(ws, params)
    wsc = ws.cpu()
    n = ref["n_qb"]

    def arr(off, count, width=1):
        a = wsc[off:off + 4 * count * width].view(torch.int32).numpy()
        return a.reshape(-1, width) if width > 1 else a

    assert h[7] == 0
    assert (h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[9]) == (
        ref["U"], P, ref["L"], n, ref["n_slots"], len(ref["combine_list"]), ref["n_workers"], ref["L0"])
    desc = arr(lay.qb_desc, n, 8)
    assert np.array_equal(desc[:, :4], ref["desc"])
    qsl, ctx = b.query_start_loc.numpy(), b.seq_lens.numpy()
    bb = ref["desc"][:, 0]
    assert np.array_equal(desc[:, 4], qsl[bb]) and np.array_equal(desc[:, 5], qsl[bb + 1] - qsl[bb])
    assert np.array_equal(desc[:, 6], ctx[bb]) and not desc[:, 7].any()
    assert np.array_equal(arr(lay.unit_prefix, n + 1), ref["unit_prefix"])
    assert np.array_equal(arr(lay.n_splits, n), ref["n_splits"])
    assert np.array_equal(arr(lay.slot_base, n), ref["slot_base"])
    assert np.array_equal(arr(lay.combine_list, len(ref["combine_list"])), ref["combine_list"])
    # and the outputs are right under this split
    compare(b, out, lse)


def test_block_mask_per_head_large():
    """A per-query-head block mask, padded with unused key-tile columns past
    64 KiB: Assign counts units from global memory (no LDS copy) and every
    Q-block unions the masks of its G heads."""
    import dataclasses
    b = W.sparse_prefill(kind="bf16", seq_len=1024)
    rng = np.random.default_rng(41)
    B_, nq = b.num_seqs, b.block_mask.shape[2]
    nk = 600                                   # 2 x 32 x 8 x 600 bytes > 64 KiB
    m = (rng.random((B_, b.num_q_heads, nq, nk)) < 0.35).astype(np.uint8)
    for t in range(nq):
        m[:, :, t, t] = 1                      # keep the diagonal
    b = dataclasses.replace(b, block_mask=torch.from_numpy(m))
    assert m.nbytes > 64 * 1024
    P = B.paged_attn_device_info(0)["default_workers"]
    ref = oracle_taskmap(b, P)
    g, out, lse, ws = gpu_run(b)
    h, lay = header(ws, params_of(g))
    assert h[7] == 0 and h[0] == ref["U"]
    up = ws.cpu()[lay.unit_prefix:lay.unit_prefix + 4 * (ref["n_qb"] + 1)].view(torch.int32).numpy()
    assert np.array_equal(up, ref["unit_prefix"])
    compare(b, out, lse)


def test_tiny_hybrid_f32():
    b = W.tiny_hybrid()
    P = B.paged_attn_device_info(0)["default_workers"]
    for kw in ({}, {"force_split_units": 1, "max_partial_slots": slots_for(b, P, 1)}, {"num_workers": 1}):
        g, out, lse, ws = gpu_run(b, **kw)
        check_no_device_error(ws, g, **kw)
        compare(b, out, lse)


def test_tiny_hybrid_closed_forms(golden):
    # Q = 0: LSE = ln(visible keys), O = mean of visible V rows
    b = W.tiny_hybrid()
    b.q = torch.zeros_like(b.q)
    g, out, lse, ws = gpu_run(b)
    counts = np.array([int(c) for _, c in golden("tiny_hybrid_visible_counts.txt")])
    assert np.abs(lse.cpu().numpy() - np.log(counts)[:, None]).max() <= 1e-5
    compare(b, out, lse)
    # one-hot V: the output row is the probability vector; masked keys get exactly 0
    b = W.tiny_hybrid()
    bt = b.block_table.numpy()
    for s in (0, 2):
        for j in range(int(b.seq_lens[s])):
            b.v_cache[bt[s, j // 16], j % 16, 0, :] = 0.0
            b.v_cache[bt[s, j // 16], j % 16, 0, j] = 1.0
    g, out, lse, ws = gpu_run(b)
    o = out.cpu().numpy()
    for t in range(2, 18):                       # chunk rows: pos = 48 + (t - 2)
        pos = 48 + (t - 2)
        assert np.all(o[t, :, pos + 1:] == 0.0)
    assert np.all(o[0, :, 37:] == 0.0)
    compare(b, out, lse)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("q_len", [1, 2, 4])
def test_decode_reduced(q_len, layout):
    b = W.splitk_decode(q_len=q_len, kv_layout=layout, batch=12, ctx_lo=100, ctx_hi=6000)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


def test_decode_mixed_mtp_and_peaked():
    b = W.splitk_decode(q_len=[1, 2, 4, 3, 1, 4, 2, 1], batch=8, ctx_lo=64, ctx_hi=5000, q_gain=8.0)
    g, out, lse, ws = gpu_run(b)
    compare(b, out, lse)


@pytest.mark.parametrize("q_len,layout", [(1, "NHD"), (4, "HND"), (2, "NHD")])
def test_decode_full_size(q_len, layout):
    """The whole split-K decode batch (64 sequences, every row), in the launch
    configuration the benchmark times."""
    b = W.splitk_decode(q_len=q_len, kv_layout=layout)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("q_len", [1, 2, 4])
@pytest.mark.parametrize("q_quant", ["token_head", "tensor"])
def test_fp8_decode_reduced(q_quant, q_len, layout):
    b = W.splitk_decode(q_len=q_len, kv_layout=layout, batch=12, ctx_lo=100, ctx_hi=6000, kind="e4m3",
                        q_quant=q_quant)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


def test_fp8_decode_page_head_kv_mixed_mtp():
    b = W.splitk_decode(q_len=[1, 2, 4, 3, 1, 4, 2, 1], batch=8, ctx_lo=64, ctx_hi=5000, kind="e4m3",
                        quant_mode="page_head", q_quant="token_head", q_gain=4.0)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


@pytest.mark.parametrize("q_len,layout", [(1, "HND"), (4, "NHD"), (1, "NHD")])
def test_fp8_decode_full_size(q_len, layout):
    b = W.splitk_decode(q_len=q_len, kv_layout=layout, kind="e4m3")
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


def test_fp8_prefill_token_head_q():
    """Per-(token, head) Q scales on the prefill path (two row blocks per lane)."""
    rng = np.random.default_rng(17)
    b = W.build_batch(rng, name="prefill_fp8_qtok", kind="e4m3", Hq=32, Hkv=8, d=128, page_size=64,
                      ctx=[700, 1100], q_len=[700, 300], quant_mode="page_head", q_quant="token_head")
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


@pytest.mark.parametrize("chunk_last", [False, True])
def test_hybrid_reduced(chunk_last):
    b = W.hybrid_chunked(batch=16, chunk=512, history=1500, dec_lo=500, dec_hi=4000, chunk_last=chunk_last)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


@pytest.mark.parametrize("chunk_last", [False, True])
def test_hybrid_full_size(chunk_last):
    """The whole hybrid step: all 575 rows (512 chunk tokens over 8192 history
    plus 63 decodes)."""
    b = W.hybrid_chunked(chunk_last=chunk_last)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


@pytest.mark.parametrize("mask", [True, False])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("mode", ["tensor", "page_head"])
def test_fp8_prefill_reduced(mode, layout, mask):
    b = W.sparse_prefill(kind="e4m3", quant_mode=mode, kv_layout=layout, mask=mask, seq_len=1024)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


def test_bf16_prefill_reduced():
    for mask in (False, True):
        b = W.sparse_prefill(kind="bf16", mask=mask, seq_len=1280)
        g, out, lse, ws = gpu_run(b)
        compare(b, out, lse)


@pytest.mark.parametrize("kind,mode,layout,mask", [("e4m3", "page_head", "HND", True),
                                                   ("e4m3", "tensor", "NHD", False),
                                                   ("bf16", None, "NHD", False)])
def test_prefill_full_size_sampled(kind, mode, layout, mask):
    b = W.sparse_prefill(kind=kind, quant_mode=mode, kv_layout=layout, mask=mask)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    rows = sample_rows(b.total_q, 40, must=(0, 1, 127, 128, 8191, 8192, 16383))
    compare(b, out, lse, rows=rows)


def test_sliding_window_reduced():
    b = W.sliding_window(seq_len=2048, window=700)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)
    # Q = 0 closed form through the kernel: LSE = ln(visible count) with landmarks
    b.q = torch.zeros_like(b.q)
    g, out, lse, ws = gpu_run(b)
    compare(b, out, lse)


@pytest.mark.parametrize("chunk", [32, 64, 128, 192])
def test_sliding_window_landmark_chunks(chunk):
    """Landmark chunks that are multiples of 64 (one landmark at most per
    64-key tile, on its last key: the lean kernel build) and one that is not
    (several per tile: the general build), each against the oracle, with Q = 0
    as well (LSE = ln of the visible-key count)."""
    b = W.sliding_window(seq_len=1600, window=600, landmark_chunk=chunk)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)
    b.q = torch.zeros_like(b.q)
    g, out, lse, ws = gpu_run(b)
    compare(b, out, lse)


def test_sliding_window_full_size_sampled(golden):
    b = W.sliding_window()
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    rows = sample_rows(b.total_q, 40, must=(0, 63, 64, 4095, 4096, 4100, 4159, 8191))
    compare(b, out, lse, rows=rows)


def test_sliding_window_decode_128k():
    b = W.sliding_window(decode=True)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)
    h = check_no_device_error(ws, g)
    # 64 window tiles x 8 kv heads = 512 units: must be split across workers
    assert h[0] == 512 and h[4] > 0
    # plain full-context decode over the same 131072 keys
    b.window, b.landmark_chunk = 0, 0
    g, out, lse, ws = gpu_run(b)
    compare(b, out, lse)


# ---------------------------------------------------------------------------
# static split (no task map) and the split policy
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 3, 8])
@pytest.mark.parametrize("kind,q_len,layout", [("bf16", 1, "NHD"), ("bf16", 4, "HND"), ("e4m3", 2, "NHD")])
def test_static_split_decode(S, kind, q_len, layout):
    b = W.splitk_decode(q_len=q_len, kv_layout=layout, batch=12, ctx_lo=100, ctx_hi=6000, kind=kind)
    g, out, lse, ws = gpu_run(b, split="static", static_splits=S)
    h = check_no_device_error(ws, g)
    assert h[3] == 12 * 8 and h[6] == 12 * 8 * S
    compare(b, out, lse)


def test_static_split_partials_follow_the_static_map():
    """Each split's partial LSE and O in its slot equal attention over exactly
    the keys the static map gives that split."""
    S = 4
    b = W.splitk_decode(q_len=2, batch=5, ctx_lo=300, ctx_hi=3000)
    g, out, lse, ws = gpu_run(b, split="static", static_splits=S)
    check_no_device_error(ws, g)
    compare(b, out, lse)
    lay = B.paged_attn_workspace_layout(params_of(g, split_mode=B.PA_SPLIT_STATIC, static_splits=S))
    D = b.head_dim
    R = lay.slot_rows
    assert R == 16                               # the static split runs the small-Q-block build
    plse = ws[lay.partial_lse:lay.partial_lse + lay.max_slots * R * 4].view(torch.float32).cpu()
    plse = plse.numpy().reshape(lay.max_slots, R)
    po = ws[lay.partial_o:lay.partial_o + lay.max_slots * R * D * 4].view(torch.float32).cpu()
    po = po.numpy().reshape(lay.max_slots, R, D)
    ctx = b.seq_lens.numpy()
    qsl = b.query_start_loc.numpy()
    G = b.num_q_heads // b.num_kv_heads
    items = taskmap.static_map(ctx, qsl, Hq=b.num_q_heads, Hkv=b.num_kv_heads, S=S)
    checked = 0
    for it, (bb, gg, t0, n) in enumerate(items):
        q = it // S
        if n == 0 or sum(1 for x in items[q * S:(q + 1) * S] if x[3]) < 2:
            continue
        kr = np.zeros((b.num_seqs, 2), np.int64)
        kr[bb] = (64 * t0, min(int(ctx[bb]), 64 * (t0 + n)))
        rows = np.zeros(b.total_q, bool)
        rows[qsl[bb]:qsl[bb + 1]] = True
        O, L = run_oracle(b, key_range=kr, rows=rows)
        for r in range((qsl[bb + 1] - qsl[bb]) * G):
            tok, head = qsl[bb] + r // G, gg * G + r % G
            assert abs(plse[it, r] - L[tok, head]) <= 1e-3
            assert np.abs(po[it, r] - O[tok, head]).max() <= 2e-2
        checked += 1
    say(f"  checked {checked} split partials")
    assert checked > 10


def test_static_split_windowed_and_full_128k_decode():
    b = W.sliding_window(decode=True)
    g, out, lse, ws = gpu_run(b, split="auto")
    mode, S = B.paged_attn_plan_split(params_of(g), b.seq_lens, b.query_start_loc)
    assert mode == B.PA_SPLIT_STATIC and S == 8
    check_no_device_error(ws, g)
    compare(b, out, lse)
    b.window, b.landmark_chunk = 0, 0
    g, out, lse, ws = gpu_run(b, split="auto")
    assert B.paged_attn_plan_split(params_of(g), b.seq_lens, b.query_start_loc) == (B.PA_SPLIT_STATIC, 64)
    check_no_device_error(ws, g)
    compare(b, out, lse)


def test_static_split_edges_and_rows_too_large():
    rng = np.random.default_rng(23)
    # empty sequences, a single key, a Q-block with fewer tiles than splits
    b = W.build_batch(rng, name="static_edges", kind="bf16", Hq=8, Hkv=2, d=128, page_size=16,
                      ctx=[1, 65, 0, 130, 7, 64, 900], q_len=[1, 3, 0, 0, 4, 2, 1], num_pages=120)
    g, out, lse, ws = gpu_run(b, split="static", static_splits=5)
    check_no_device_error(ws, g)
    compare(b, out, lse)
    # a sequence whose rows do not fit one small Q-block: reported, other rows still right
    b = W.build_batch(rng, name="static_too_big", kind="bf16", Hq=8, Hkv=2, d=64, page_size=64,
                      ctx=[300, 200, 500], q_len=[1, 5, 2], num_pages=20)
    g, out, lse, ws = gpu_run(b, split="static", static_splits=2)
    h, _ = header(ws, params_of(g))
    assert h[7] == 6
    rows = np.ones(b.total_q, bool)
    rows[1:6] = False
    compare(b, out, lse, rows=rows)


def test_decode_kernel_choice_by_q_len_bound():
    """Decode batches run the small-Q-block kernel when the caller states
    max_q_len (run_batch passes the batch's own); the general kernel, chosen
    without the bound, gives the same result; a bound below a sequence's
    q_len is reported."""
    b = W.splitk_decode(q_len=[1, 2, 4, 3, 1, 4, 2, 1], batch=8, ctx_lo=64, ctx_hi=5000)
    assert b.max_q_len == 4
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)
    g, out2, lse2, ws2 = gpu_run(b, max_q_len=0)
    check_no_device_error(ws2, g)
    compare(b, out2, lse2)
    g, out3, lse3, ws3 = gpu_run(b, max_q_len=2)
    h, _ = header(ws3, params_of(g))
    assert h[7] == 7
    # a prefill batch with a small bound: refused on the device, not computed as decode
    rng = np.random.default_rng(3)
    b = W.build_batch(rng, name="hint_prefill", kind="bf16", Hq=8, Hkv=2, d=64, page_size=64,
                      ctx=[300, 200], q_len=[100, 1], num_pages=10)
    g, out4, lse4, ws4 = gpu_run(b, max_q_len=1, min_q_len=0)
    h, _ = header(ws4, params_of(g))
    assert h[7] == 7
    # ... and a lower bound above a sequence's q_len
    g, out5, lse5, ws5 = gpu_run(b, max_q_len=0, min_q_len=100)
    h, _ = header(ws5, params_of(g))
    assert h[7] == 7


@pytest.mark.parametrize("kind", ["bf16", "e4m3"])
def test_prefill_kernel_choice_by_q_len_bound(kind):
    """Prefill batches run the large-Q-block kernel when the caller states
    min_q_len (run_batch passes the batch's own); the general kernel agrees."""
    rng = np.random.default_rng(12)
    b = W.build_batch(rng, name=f"prefill_bound_{kind}", kind=kind, Hq=32, Hkv=8, d=128, page_size=64,
                      ctx=[900, 1500, 700], q_len=[900, 400, 0], quant_mode="tensor" if kind == "e4m3" else None)
    assert b.min_q_len == 400
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)
    g, out2, lse2, ws2 = gpu_run(b, min_q_len=0, max_q_len=0)
    check_no_device_error(ws2, g)
    compare(b, out2, lse2)


@pytest.mark.parametrize("kind,mode", [("bf16", None), ("e4m3", "tensor"), ("e4m3", "page_head")])
def test_large_qblocks_ragged_tails_poisoned(kind, mode):
    """Large-Q-block runs (the lean build: d 128, 64-token pages, no block
    mask) whose sequences end inside a 64-key tile, with every cache slot past
    the ends poisoned (NaN in bf16, 0x7F in FP8), whole and chunked prefill
    mixed: the keys past an end are zeroed in LDS and masked, so no poison
    reaches O or the LSE."""
    rng = np.random.default_rng(21)
    b = W.build_batch(rng, name=f"ragged_large_{kind}_{mode}", kind=kind, Hq=32, Hkv=8, d=128, page_size=64,
                      ctx=[1000, 1537, 130, 777], q_len=[1000, 600, 130, 777], quant_mode=mode, poison=True)
    assert b.min_q_len == 130
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


@pytest.mark.parametrize("kind", ["bf16", "e4m3"])
def test_large_qblock_segment_over_one_tile_chunk(kind):
    """A worker segment longer than the 1024-tile chunk the large-Q-block loop
    takes at once (forced split of 4096 units per worker over a 70,000-key
    context): the K/V pipeline restarts at the chunk boundary, and the result
    still matches the oracle (sampled rows)."""
    rng = np.random.default_rng(33)
    b = W.build_batch(rng, name=f"long_segment_{kind}", kind=kind, Hq=32, Hkv=8, d=128, page_size=64,
                      ctx=[70000], q_len=[32], quant_mode="tensor" if kind == "e4m3" else None)
    P = B.paged_attn_device_info(0)["default_workers"]
    force = 4096
    g, out, lse, ws = gpu_run(b, force_split_units=force, max_partial_slots=slots_for(b, P, force))
    h = check_no_device_error(ws, g, force_split_units=force, max_partial_slots=slots_for(b, P, force))
    assert h[2] == force
    compare(b, out, lse, rows=sample_rows(b.total_q, 12, must=(0, 31)))


def test_sliding_window_ragged_tail_poisoned():
    """The sliding-window forward (landmarks every 64 keys: the lean build)
    over a sequence that ends inside a tile, its pages' free slots poisoned."""
    b = W.sliding_window(seq_len=1000, window=300)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


@pytest.mark.parametrize("make,kw", [
    (lambda: W.splitk_decode(q_len=1, batch=16, ctx_lo=64, ctx_hi=6000), {}),
    (lambda: W.splitk_decode(q_len=[1, 2, 4, 3] * 4, batch=16, ctx_lo=64, ctx_hi=6000), {"max_q_len": 0}),
    (lambda: W.hybrid_chunked(batch=12, chunk=300, history=900, dec_lo=100, dec_hi=3000), {}),
    (lambda: W.sparse_prefill(kind="e4m3", seq_len=1024), {"force_split_units": 3}),
    (lambda: W.sparse_prefill(kind="bf16", seq_len=1000, mask=False), {"force_split_units": 3}),
    (lambda: W.sparse_prefill(kind="e4m3", seq_len=1000, mask=False), {"force_split_units": 5}),
    (lambda: W.sliding_window(seq_len=1500, window=512), {"force_split_units": 4}),
    (lambda: W.sliding_window(decode=True), {"split": "static", "static_splits": 8}),
    (lambda: W.build_batch(np.random.default_rng(8), name="empty_qblocks", kind="bf16", Hq=8, Hkv=2, d=64,
                           page_size=16, ctx=[40, 300, 90], q_len=[3, 300, 2], num_pages=40, window=1,
                           landmark_chunk=2, window_expand_to_chunk=False), {}),
], ids=["decode", "mtp_general", "hybrid", "fp8_forced", "lean_bf16_forced", "lean_fp8_forced", "lean_window_forced",
        "static", "empty"])
def test_fused_combine_equals_combine_kernel(make, kw):
    """The fused merge (last finisher of a split Q-block) runs the same
    arithmetic in the same order as the Combine kernel: bit-identical."""
    b = make()
    if "force_split_units" in kw:
        kw = dict(kw, max_partial_slots=slots_for(b, B.paged_attn_device_info(0)["default_workers"],
                                                  kw["force_split_units"]))
    g, o1, l1, ws1 = gpu_run(b, fused_combine=True, **kw)
    check_no_device_error(ws1, g)
    g, o2, l2, ws2 = gpu_run(b, **kw)
    check_no_device_error(ws2, g)
    assert torch.equal(o1.view(torch.uint8) if o1.dtype != torch.float32 else o1.view(torch.int32),
                       o2.view(torch.uint8) if o2.dtype != torch.float32 else o2.view(torch.int32))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    if b.total_q <= 4096:
        compare(b, o1, l1)


@pytest.mark.parametrize("split", ["dynamic", "static"])
def test_graph_replay_with_changing_batch(split):
    """One forward call captured in a HIP graph, replayed after the batch
    metadata (seq_lens, query_start_loc, block table) is rewritten in place:
    every replay equals an eager call on the same data bit for bit and
    matches the oracle; eager work and synchronisation run between replays."""
    vs = W.replay_variants()
    g0 = vs[0].to(DEV)
    P = B.paged_attn_device_info(0)["default_workers"]
    bt, sl, qsl = g0.block_table.clone(), g0.seq_lens.clone(), g0.query_start_loc.clone()
    kw = dict(softmax_scale=g0.softmax_scale, kv_layout=g0.kv_layout, causal=True, max_q_len=4, num_workers=P)
    if split == "static":
        kw.update(split="static", static_splits=4)
    out = torch.empty((g0.total_q, g0.num_q_heads, g0.head_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((g0.total_q, g0.num_q_heads), dtype=torch.float32, device=DEV)
    _, _, ws = B.paged_attn_fwd(g0.q, g0.k_cache, g0.v_cache, bt, sl, qsl, None, g0.scales, out, lse, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.paged_attn_fwd(g0.q, g0.k_cache, g0.v_cache, bt, sl, qsl, None, g0.scales, out, lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    ws_eager = torch.empty_like(ws)
    for rep in range(2):
        for v in vs[1:] + vs[:1]:
            bt.copy_(v.block_table.to(DEV))
            sl.copy_(v.seq_lens.to(DEV))
            qsl.copy_(v.query_start_loc.to(DEV))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            o_r, l_r = out.clone(), lse.clone()
            check_no_device_error(ws, g0)
            o_e, l_e, _ = B.paged_attn_fwd(g0.q, g0.k_cache, g0.v_cache, bt, sl, qsl, None, g0.scales,
                                           workspace=ws_eager, **kw)
            torch.cuda.synchronize()
            assert torch.equal(o_r.view(torch.int16), o_e.view(torch.int16))
            assert torch.equal(l_r.view(torch.int32), l_e.view(torch.int32))
            if rep == 0:
                compare(v, o_r, l_r)


def test_small_kernel_with_block_mask_and_f32_static():
    """Decode rows under a block mask (small Q-blocks on the masked segment
    path of the small-Q-block kernel), and fp32 decode under a static split
    and the fused merge (fp32 outputs)."""
    rng = np.random.default_rng(31)
    b = W.build_batch(rng, name="decode_mask", kind="bf16", Hq=32, Hkv=8, d=128, page_size=64,
                      ctx=[3000, 700, 1800, 129], q_len=[1, 2, 4, 1], block_mask_skip=0.5)
    assert b.max_q_len * 4 <= 16
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)
    rng = np.random.default_rng(32)
    b = W.build_batch(rng, name="decode_f32", kind="f32", Hq=4, Hkv=1, d=64, page_size=16,
                      ctx=[37, 300, 1000, 64], q_len=[1, 4, 2, 0], num_pages=120)
    for kw in ({"split": "static", "static_splits": 3}, {"split": "static", "static_splits": 3, "fused_combine": True},
               {"force_split_units": 2, "max_partial_slots": 512, "fused_combine": True}):
        g, out, lse, ws = gpu_run(b, **kw)
        check_no_device_error(ws, g)
        compare(b, out, lse)


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_small_pages(d):
    """FP8 with 16-token pages (tiles span four pages: the register-staged
    prefill path and per-key page lookups), prefill rows and decode rows."""
    rng = np.random.default_rng(41 + d)
    b = W.build_batch(rng, name=f"fp8_pages16_d{d}", kind="e4m3", Hq=8, Hkv=2, d=d, page_size=16,
                      ctx=[700, 300, 90], q_len=[300, 1, 4], quant_mode="tensor", q_quant="token_head")
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


@pytest.mark.parametrize("kind,d,page_size,layout,quant,Hq,Hkv,qmax", [
    ("e4m3", 64, 64, "NHD", "tensor", 16, 4, 4),
    ("e4m3", 64, 64, "HND", "page_head", 32, 8, 2),
    ("e4m3", 64, 16, "NHD", "tensor", 16, 4, 3),
    ("e4m3", 128, 16, "HND", "tensor", 32, 8, 2),
    ("bf16", 64, 64, "NHD", None, 16, 4, 4),
    ("bf16", 64, 16, "HND", None, 32, 8, 1),
])
def test_sequence_qblocks_head_dims_and_pages(kind, d, page_size, layout, quant, Hq, Hkv, qmax):
    """Decode with sequence Q-blocks (every query head of a sequence in one
    block) at d = 64 and with 16-token pages, where the fp8 K rows and Q rows
    are read in the paired dim order (two K-steps per 16-byte read) through
    both the page-window and the per-key row lookups; ragged contexts end
    mid-tile."""
    rng = np.random.default_rng(300 + d + page_size + Hkv)
    nb = 10
    ctx = rng.integers(40, 3000, size=nb)
    q_len = rng.integers(1, qmax + 1, size=nb)
    b = W.build_batch(rng, name=f"seqqb_{kind}_d{d}_p{page_size}_{layout}", kind=kind, Hq=Hq, Hkv=Hkv, d=d,
                      page_size=page_size, ctx=ctx, q_len=q_len, kv_layout=layout, quant_mode=quant,
                      q_quant="token_head" if kind == "e4m3" else "tensor")
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)


def test_auto_policy_runs_each_shape():
    for b in (W.splitk_decode(q_len=1, batch=12, ctx_lo=100, ctx_hi=6000),
              W.build_batch(np.random.default_rng(5), name="uniform", kind="bf16", Hq=32, Hkv=8, d=128,
                            page_size=64, ctx=[2048] * 64, q_len=[1] * 64),
              W.hybrid_chunked(batch=8, chunk=256, history=700, dec_lo=300, dec_hi=2000)):
        g, out, lse, ws = gpu_run(b, split="auto")
        check_no_device_error(ws, g)
        compare(b, out, lse)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_page_permutation_bitwise():
    b = W.splitk_decode(q_len=2, batch=6, ctx_lo=100, ctx_hi=3000)
    _, o1, l1, _ = gpu_run(b)
    rng = np.random.default_rng(5)
    pi = torch.from_numpy(rng.permutation(b.num_pages))
    k2, v2 = torch.empty_like(b.k_cache), torch.empty_like(b.v_cache)
    k2[pi], v2[pi] = b.k_cache, b.v_cache
    bt = b.block_table.clone()
    m = bt >= 0
    bt[m] = pi[bt[m].long()].to(torch.int32)
    b.k_cache, b.v_cache, b.block_table = k2, v2, bt
    _, o2, l2, _ = gpu_run(b)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_nhd_equals_hnd_bitwise_and_deterministic():
    a = W.splitk_decode(q_len=4, kv_layout="NHD", batch=6, ctx_lo=100, ctx_hi=3000)
    c = W.splitk_decode(q_len=4, kv_layout="HND", batch=6, ctx_lo=100, ctx_hi=3000)
    _, oa, la, _ = gpu_run(a)
    _, oc, lc, _ = gpu_run(c)
    assert torch.equal(oa, oc) and torch.equal(la, lc)
    _, oa2, la2, _ = gpu_run(a)
    assert torch.equal(oa, oa2) and torch.equal(la, la2)
    p = W.sparse_prefill(kind="e4m3", quant_mode="page_head", kv_layout="NHD", seq_len=512)
    p2 = W.sparse_prefill(kind="e4m3", quant_mode="page_head", kv_layout="HND", seq_len=512)
    _, o1, l1, _ = gpu_run(p)
    _, o2, l2, _ = gpu_run(p2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_forced_split_matches_natural():
    b = W.hybrid_chunked(batch=8, chunk=300, history=900, dec_lo=200, dec_hi=3000)
    _, o1, l1, _ = gpu_run(b)
    P = B.paged_attn_device_info(0)["default_workers"]
    _, o2, l2, _ = gpu_run(b, force_split_units=1, max_partial_slots=slots_for(b, P, 1))
    assert (o1.float() - o2.float()).abs().max() <= 2e-2
    assert (l1 - l2).abs().max() <= 1e-3
    compare(b, o2, l2)


def test_edge_cases():
    rng = np.random.default_rng(17)
    # empty q_len sequences, single-key sequences, keys not a multiple of 64, one page per key
    b = W.build_batch(rng, name="edges", kind="bf16", Hq=8, Hkv=2, d=128, page_size=16,
                      ctx=[1, 65, 0, 130, 7, 64], q_len=[1, 3, 0, 0, 7, 40], num_pages=40)
    g, out, lse, ws = gpu_run(b)
    check_no_device_error(ws, g)
    compare(b, out, lse)
    # a window so narrow that landmark-only tiles appear; a row with no visible key
    b = W.build_batch(rng, name="narrow", kind="bf16", Hq=4, Hkv=1, d=64, page_size=64,
                      ctx=[300], q_len=[300], window=1, landmark_chunk=2, window_expand_to_chunk=False)
    g, out, lse, ws = gpu_run(b)
    O, L = run_oracle(b)
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    empty = ~np.isfinite(L)
    assert empty.any()
    assert np.all(l[empty] == -np.inf) and np.all(o[empty] == 0)
    assert np.abs(o[~empty] - O[~empty]).max() <= 2e-2
    assert np.abs(l[~empty] - L[~empty]).max() <= 1e-3
    # non-causal attention
    b = W.splitk_decode(q_len=3, batch=4, ctx_lo=70, ctx_hi=500)
    g, out, lse, ws = gpu_run(b, causal=False)
    compare(b, out, lse, causal=False)


@pytest.mark.parametrize("make", [
    lambda: W.splitk_decode(q_len=[1, 2, 4, 3] * 3, batch=12, ctx_lo=64, ctx_hi=3000),
    lambda: W.hybrid_chunked(batch=6, chunk=200, history=700, dec_lo=100, dec_hi=2000),
], ids=["mtp_mix", "hybrid"])
def test_strided_views_bitwise(make):
    """Q as the head slice of a fused QKV buffer, the block table as the
    leading columns of a wider table, O as a slice of wider rows and LSE with
    a column stride of 2: the same bits as with contiguous tensors, and the
    padding between the views' elements left untouched."""
    import dataclasses
    b = make()
    g, o1, l1, _ = gpu_run(b)
    T, Hq, d = g.q.shape
    Hkv, mp = g.num_kv_heads, g.block_table.shape[1]
    qkv = torch.zeros((T, Hq + 2 * Hkv, d), dtype=g.q.dtype, device=DEV)
    qkv[:, :Hq] = g.q
    bt = torch.full((g.num_seqs, mp + 37), -1, dtype=torch.int32, device=DEV)
    bt[:, :mp] = g.block_table
    gs = dataclasses.replace(g, q=qkv[:, :Hq], block_table=bt[:, :mp])
    ob = torch.full((T, Hq, d + 64), 7.0, dtype=o1.dtype, device=DEV)
    lb = torch.full((T, 2 * Hq + 3), 7.0, dtype=torch.float32, device=DEV)
    o2, l2 = ob[:, :, :d], lb[:, 1:1 + 2 * Hq:2]
    say(f"  launch {b.name} strided q {tuple(gs.q.stride())} bt {tuple(gs.block_table.stride())} "
        f"out {tuple(o2.stride())} lse {tuple(l2.stride())}")
    B.run_batch(gs, out=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.contiguous().view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.contiguous().view(torch.int32))
    assert (ob[:, :, d:] == 7.0).all()
    assert (lb[:, 0] == 7.0).all() and (lb[:, 2:2 * Hq + 1:2] == 7.0).all() and (lb[:, 2 * Hq + 1:] == 7.0).all()
    compare(b, o2, l2)


# GQA ratios other than the 8B shape's G = 4.  (Hq, Hkv) per G; the mixed batch
# holds decode rows with MTP (q_len 1/2/4) and a prefill chunk, so small and
# large Q-blocks of every ratio run in one launch; G = 16 at q_len 1 is a
# Q-block of exactly 16 rows, G = 32 sends even single-token rows to the
# 128-row path (4 tokens per Q-block).
_GQA = {1: (8, 8), 2: (16, 8), 8: (32, 4), 16: (32, 2), 32: (32, 1)}


@pytest.mark.parametrize("kind", ["bf16", "e4m3"])
@pytest.mark.parametrize("G", sorted(_GQA))
def test_gqa_ratios(G, kind):
    Hq, Hkv = _GQA[G]
    qm = "tensor" if kind == "e4m3" else None
    rng = np.random.default_rng(100 + G)
    mixed = W.build_batch(rng, name=f"gqa{G}_{kind}_mixed", kind=kind, Hq=Hq, Hkv=Hkv, d=128, page_size=64,
                          ctx=[300, 1200, 2500, 77, 700, 64], q_len=[1, 2, 4, 1, 150, 0], quant_mode=qm)
    g, out, lse, ws = gpu_run(mixed)
    check_no_device_error(ws, g)
    compare(mixed, out, lse)
    # every worker holding two units: many Q-blocks split, merged by Combine
    P = B.paged_attn_device_info(0)["default_workers"]
    g, out, lse, ws = gpu_run(mixed, force_split_units=2, max_partial_slots=slots_for(mixed, P, 2))
    check_no_device_error(ws, g)
    compare(mixed, out, lse)
    # decode only: the small-Q-block build when max_q_len * G <= 16, else the
    # general one; then a static split, which needs q_len * G <= 16
    ql = [1, 1, 1, 1, 1] if G >= 8 else [1, 2, 4, 1, 3]
    dec = W.build_batch(np.random.default_rng(200 + G), name=f"gqa{G}_{kind}_decode", kind=kind, Hq=Hq,
                        Hkv=Hkv, d=128, page_size=64, ctx=[300, 1200, 2500, 77, 4100], q_len=ql, quant_mode=qm)
    g, out, lse, ws = gpu_run(dec)
    check_no_device_error(ws, g)
    compare(dec, out, lse)
    g, out, lse, ws = gpu_run(dec, split="static", static_splits=3)
    h, _ = header(ws, params_of(g, split_mode=B.PA_SPLIT_STATIC, static_splits=3))
    if max(ql) * G <= 16:
        assert h[7] == 0, f"device error word {h[7]}"
        compare(dec, out, lse)
    else:
        assert h[7] == 6                          # PA_DEV_STATIC_ROWS: a Q-block beyond 16 rows



# Sequence Q-blocks: a decode batch whose kv heads split over the four waves
# (Hkv % 4 == 0, q_len * G * Hkv / 4 <= 16) gets one Q-block per sequence with
# every query head; units are (tile, kv head) pairs and each wave owns Hkv / 4
# kv heads.  Checked against the oracle and against one Q-block per kv head.
@pytest.mark.parametrize("kind,layout", [("bf16", "NHD"), ("bf16", "HND"), ("e4m3", "NHD"), ("e4m3", "HND")])
@pytest.mark.parametrize("q_len", [1, [1, 2, 0, 2]])
def test_sequence_qblocks_decode(kind, layout, q_len):
    b = W.splitk_decode(q_len=q_len if isinstance(q_len, int) else q_len * 5, batch=20, ctx_lo=40, ctx_hi=5000,
                        kv_layout=layout, kind=kind, q_gain=4.0)
    assert sequence_qblocks(b)
    P = B.paged_attn_device_info(0)["default_workers"]
    for kw in ({}, {"num_workers": 37}, {"force_split_units": 1}, {"force_split_units": 3, "fused_combine": True}):
        if "force_split_units" in kw:
            kw = dict(kw, max_partial_slots=slots_for(b, kw.get("num_workers") or P, kw["force_split_units"]))
        g, out, lse, ws = gpu_run(b, **kw)
        check_no_device_error(ws, g)
        compare(b, out, lse)
    # the per-kv-head Q-blocks of the same batch agree within the tolerance
    g, o2, l2, ws2 = gpu_run(b, qblock_per_kv_head=True)
    check_no_device_error(ws2, g)
    to, tl = TOL[b.kind]
    assert (o2.float() - out.float()).abs().max().item() <= to and (l2 - lse).abs().max().item() <= tl


def test_sequence_qblocks_window_and_short_sequences():
    """Windowed decode with landmarks, sequences shorter than a tile and a
    q_len 0 sequence, under the dynamic split."""
    rng = np.random.default_rng(31)
    b = W.build_batch(rng, name="seqqb_window", kind="bf16", Hq=32, Hkv=8, d=128, page_size=64,
                      ctx=[3, 64, 65, 700, 4100, 90, 1], q_len=[1, 1, 2, 2, 1, 0, 1], window=300,
                      landmark_chunk=64)
    assert sequence_qblocks(b)
    for kw in ({}, {"force_split_units": 2, "max_partial_slots": 4096}):
        g, out, lse, ws = gpu_run(b, **kw)
        check_no_device_error(ws, g)
        compare(b, out, lse)
