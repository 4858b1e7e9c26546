"""Pins for oracle.attention: what the pages and the mathematics fix, checked
against code that shares nothing with the oracle's vectorised path."""
import math

import numpy as np
import pytest
import torch

from attention_paged_kv_attn_amd import workloads as W
from oracle import brute
from oracle.attention import paged_attention, visible
from tests.oracle_helpers import dequant64, run_oracle, stored_np


def _q_scale64(batch):
    """The Q scale as a float or a [total_q, Hq, 1] array, widened by torch."""
    if batch.scales is None:
        return None
    if batch.scales.get("q_mode", "tensor") == "tensor":
        return float(batch.scales["q"][0])
    return batch.scales["q"].to(torch.float64).numpy()[:, :, None]


def _dense_lists(batch, scales_per_seq=None):
    q = dequant64(batch.q, _q_scale64(batch)).tolist()
    ks, vs = [], []
    for b, (k, v) in enumerate(zip(batch.dense_k, batch.dense_v)):
        if batch.scales is None:
            ks.append(dequant64(k).tolist())
            vs.append(dequant64(v).tolist())
        else:
            ks.append(dequant64(k, scales_per_seq[b]["k"]).tolist())
            vs.append(dequant64(v, scales_per_seq[b]["v"]).tolist())
    return q, ks, vs


def _brute(batch, **kw):
    sc = None
    if batch.scales is not None:
        sc = []
        bt = batch.block_table.numpy()
        for b, ctx in enumerate(batch.seq_lens.tolist()):
            per = {}
            for which in ("k", "v"):
                s = batch.scales[which].numpy().astype(np.float64)
                if batch.scales["mode"] == "tensor":
                    per[which] = float(s[0])
                else:
                    pages = bt[b, np.arange(ctx) // batch.page_size]
                    per[which] = s[pages][:, :, None]          # [ctx, Hkv, 1]
            sc.append(per)
    q, ks, vs = _dense_lists(batch, sc)
    args = dict(Hq=batch.num_q_heads, scale=batch.softmax_scale, causal=batch.causal,
                window=batch.window, expand_to_chunk=batch.window_expand_to_chunk,
                chunk=batch.landmark_chunk, tile=batch.block_mask_tile,
                block_mask=None if batch.block_mask is None else batch.block_mask.numpy().tolist())
    args.update(kw)
    O, L = brute.attention_batch(q, ks, vs, batch.seq_lens.tolist(), batch.query_start_loc.tolist(), **args)
    return np.array(O), np.array(L)


def test_brute_force_tiny_hybrid():
    b = W.tiny_hybrid()
    O, L = run_oracle(b)
    Ob, Lb = _brute(b)
    assert np.abs(O - Ob).max() <= 1e-12
    assert np.abs(L - Lb).max() <= 1e-12


@pytest.mark.parametrize("mode", ["tensor", "page_head"])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("q_quant", ["tensor", "token_head"])
def test_brute_force_fp8(mode, layout, q_quant):
    rng = np.random.default_rng(41)
    b = W.build_batch(rng, name="tiny_fp8", kind="e4m3", Hq=4, Hkv=2, d=32, page_size=16,
                      ctx=[40, 70], q_len=[1, 20], num_pages=12, quant_mode=mode, keep_dense=True,
                      kv_layout=layout, q_quant=q_quant)
    O, L = run_oracle(b)
    Ob, Lb = _brute(b)
    assert np.abs(O - Ob).max() <= 1e-12
    assert np.abs(L - Lb).max() <= 1e-12


def test_token_head_q_scale_reduces_to_per_tensor():
    """Per-(token, head) Q scales that are all equal give the per-tensor result
    bit for bit; scaling one (token, head) entry changes that row only."""
    rng = np.random.default_rng(43)
    b = W.build_batch(rng, name="tiny_fp8_q", kind="e4m3", Hq=8, Hkv=2, d=32, page_size=16,
                      ctx=[33, 90, 17], q_len=[1, 4, 2], num_pages=16, quant_mode="tensor",
                      q_quant="tensor")
    c = float(b.scales["q"][0])
    total_q, Hq = b.q.shape[:2]
    O1, L1 = run_oracle(b)
    sc = {"mode": "tensor", "q_mode": "token_head", "q": np.full((total_q, Hq), c, np.float32),
          "k": float(b.scales["k"][0]), "v": float(b.scales["v"][0])}
    O2, L2 = run_oracle(b, scales=sc)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    sc["q"] = sc["q"].copy()
    sc["q"][3, 5] *= 4.0
    O3, L3 = run_oracle(b, scales=sc)
    changed = np.zeros((total_q, Hq), dtype=bool)
    changed[3, 5] = True
    assert np.array_equal(O3[~changed], O1[~changed]) and np.array_equal(L3[~changed], L1[~changed])
    assert not np.allclose(O3[3, 5], O1[3, 5])
    # a Q scale of c * 4 on one row is the same as a softmax scale four times as large there
    O4, L4 = run_oracle(b, softmax_scale=4.0 * b.softmax_scale)
    assert np.abs(O3[3, 5] - O4[3, 5]).max() <= 1e-12 and abs(L3[3, 5] - L4[3, 5]) <= 1e-12


def _sdpa_check(batch):
    """torch SDPA in float64 per (sequence, head) with a mask from brute.is_visible."""
    O, _ = run_oracle(batch)
    G = batch.num_q_heads // batch.num_kv_heads
    qsl = batch.query_start_loc.tolist()
    q64 = torch.from_numpy(dequant64(batch.q, _q_scale64(batch)))
    worst = 0.0
    for b, ctx in enumerate(batch.seq_lens.tolist()):
        q0, q1 = qsl[b], qsl[b + 1]
        ql = q1 - q0
        k = torch.from_numpy(dequant64(batch.dense_k[b]))
        v = torch.from_numpy(dequant64(batch.dense_v[b]))
        for h in range(batch.num_q_heads):
            mrow = None
            if batch.block_mask is not None:
                bm = batch.block_mask.numpy()
                mrow = bm[b, 0 if bm.shape[1] == 1 else h]
            mask = torch.tensor([[brute.is_visible(ctx - ql + i, j, ctx, causal=batch.causal,
                                                   window=batch.window,
                                                   expand_to_chunk=batch.window_expand_to_chunk,
                                                   chunk=batch.landmark_chunk, mask=mrow,
                                                   tile=batch.block_mask_tile)
                                  for j in range(ctx)] for i in range(ql)])
            ref = torch.nn.functional.scaled_dot_product_attention(
                q64[q0:q1, h][None], k[:, h // G][None], v[:, h // G][None], attn_mask=mask[None],
                scale=batch.softmax_scale)[0]
            worst = max(worst, float((ref - torch.from_numpy(O[q0:q1, h])).abs().max()))
    return worst


def test_sdpa_tiny_hybrid():
    assert _sdpa_check(W.tiny_hybrid()) <= 1e-12


def test_sdpa_reduced_hybrid_chunked():
    rng = np.random.default_rng(3)
    b = W.build_batch(rng, name="hyb_small", kind="bf16", Hq=8, Hkv=2, d=64, page_size=64,
                      ctx=[64 + 40, 150, 300, 77], q_len=[40, 1, 1, 1], keep_dense=True)
    assert _sdpa_check(b) <= 1e-12


def test_sdpa_reduced_sparse_prefill():
    rng = np.random.default_rng(4)
    b = W.build_batch(rng, name="sparse_small", kind="bf16", Hq=4, Hkv=2, d=32, page_size=64,
                      ctx=[512, 384], q_len=[512, 384], keep_dense=True, block_mask_skip=0.6)
    assert _sdpa_check(b) <= 1e-12


def test_sdpa_reduced_sliding_window():
    rng = np.random.default_rng(5)
    b = W.build_batch(rng, name="win_small", kind="bf16", Hq=2, Hkv=1, d=32, page_size=64,
                      ctx=[400], q_len=[400], identity_pages=True, keep_dense=True,
                      window=100, landmark_chunk=32)
    assert _sdpa_check(b) <= 1e-12


def _zero_q(batch):
    batch.q = torch.zeros_like(batch.q)
    return batch


def test_q_zero_closed_form_counts(golden):
    b = _zero_q(W.tiny_hybrid())
    O, L = run_oracle(b)
    counts = {int(r): int(c) for r, c in golden("tiny_hybrid_visible_counts.txt")}
    for row, c in counts.items():
        assert np.abs(L[row] - math.log(c)).max() <= 1e-12
    # O is the mean of the visible V rows
    qsl = b.query_start_loc.tolist()
    for s, ctx in enumerate(b.seq_lens.tolist()):
        v = dequant64(b.dense_v[s])[:, 0, :]              # Hkv = 1
        for t in range(qsl[s], qsl[s + 1]):
            want = v[:counts[t]].mean(axis=0)
            assert np.abs(O[t] - want[None]).max() <= 1e-12


def test_sliding_window_visible_counts(golden):
    for pos, expand, want in golden("sliding_window_counts.txt"):
        pos, expand, want = int(pos), bool(int(expand)), int(want)
        ctx = pos + 1
        n = visible(np.array([pos]), np.arange(ctx), ctx, causal=True, window=4096,
                    expand_to_chunk=expand, landmark_chunk=64).sum()
        assert n == want, (pos, expand)
    # and through the whole pipeline (Q = 0 -> LSE = ln count) on sampled rows
    b = _zero_q(W.sliding_window(seq_len=8192))
    rows = np.zeros(b.total_q, dtype=bool)
    picks = {0: 1, 63: 63, 64: 64, 4095: 4032, 4096: 4033, 4100: 4037, 4159: 4032, 8191: 4032}
    rows[list(picks)] = True
    _, L = run_oracle(b, rows=rows)
    for pos, want in picks.items():
        assert np.abs(L[pos] - math.log(want)).max() <= 1e-12


def test_one_hot_v_gives_probabilities():
    b = W.tiny_hybrid()
    bt = b.block_table.numpy()
    # sequence 0 (37 keys) and sequence 2 (64 keys): V[j] = e_j  (d = 64)
    for s in (0, 2):
        ctx = int(b.seq_lens[s])
        for j in range(ctx):
            b.v_cache[bt[s, j // 16], j % 16, 0, :] = 0.0
            b.v_cache[bt[s, j // 16], j % 16, 0, j] = 1.0
    O, L = run_oracle(b)
    qsl = b.query_start_loc.tolist()
    q = dequant64(b.q)
    for s in (0, 2):
        ctx = int(b.seq_lens[s])
        k = dequant64(b.dense_k[s])[:, 0, :]
        ql = qsl[s + 1] - qsl[s]
        for t in range(qsl[s], qsl[s + 1]):
            pos = ctx - ql + (t - qsl[s])
            for h in range(4):
                p = O[t, h]
                assert np.all(p[pos + 1:] == 0.0)            # masked keys: exactly zero weight
                scores = [sum(a * c for a, c in zip(q[t, h], k[j])) * b.softmax_scale for j in range(pos + 1)]
                m = max(scores)
                z = sum(math.exp(x - m) for x in scores)
                want = [math.exp(x - m) / z for x in scores]
                assert np.abs(p[:pos + 1] - want).max() <= 1e-12
                # LSE identity: sum_j exp(s_j - LSE) = 1
                assert abs(sum(math.exp(x - L[t, h]) for x in scores) - 1.0) <= 1e-12


def test_single_visible_key_and_constant_v():
    rng = np.random.default_rng(7)
    b = W.build_batch(rng, name="c", kind="bf16", Hq=4, Hkv=2, d=32, page_size=64,
                      ctx=[130], q_len=[130], keep_dense=True)
    O, L = run_oracle(b)
    q = dequant64(b.q)
    k = dequant64(b.dense_k[0])
    v = dequant64(b.dense_v[0])
    for h in range(4):
        assert np.array_equal(O[0, h], v[0, h // 2])                      # pos 0 sees key 0 only
        assert abs(L[0, h] - float(q[0, h] @ k[0, h // 2]) * b.softmax_scale) <= 1e-12
    # constant V: every output row is that constant
    const = torch.tensor(np.linspace(-2, 2, 32), dtype=torch.bfloat16)
    b.v_cache[:] = const
    O2, L2 = run_oracle(b)
    assert np.abs(O2 - dequant64(const)[None, None]).max() <= 1e-14
    assert np.array_equal(L2, L)


def test_page_permutation_invariance():
    b = W.tiny_hybrid()
    O, L = run_oracle(b)
    rng = np.random.default_rng(99)
    pi = torch.from_numpy(rng.permutation(b.num_pages))
    k2 = torch.empty_like(b.k_cache)
    v2 = torch.empty_like(b.v_cache)
    k2[pi] = b.k_cache
    v2[pi] = b.v_cache
    bt = b.block_table.clone()
    valid = bt >= 0
    bt[valid] = pi[bt[valid].long()].to(torch.int32)
    b.k_cache, b.v_cache, b.block_table = k2, v2, bt
    O2, L2 = run_oracle(b)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_nhd_equals_hnd():
    a = W.splitk_decode(q_len=2, kv_layout="NHD", batch=4, ctx_lo=70, ctx_hi=400)
    c = W.splitk_decode(q_len=2, kv_layout="HND", batch=4, ctx_lo=70, ctx_hi=400)
    Oa, La = run_oracle(a)
    Oc, Lc = run_oracle(c)
    assert np.array_equal(Oa, Oc) and np.array_equal(La, Lc)


def test_gqa_equals_replicated_mha():
    b = W.splitk_decode(q_len=4, batch=3, ctx_lo=64, ctx_hi=300)
    O, L = run_oracle(b)
    G = b.num_q_heads // b.num_kv_heads
    b.k_cache = b.k_cache.repeat_interleave(G, dim=2)
    b.v_cache = b.v_cache.repeat_interleave(G, dim=2)
    b.num_kv_heads = b.num_q_heads
    O2, L2 = run_oracle(b)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_wide_window_without_landmarks_is_causal():
    b = W.tiny_hybrid()
    O, L = run_oracle(b)
    O2, L2 = run_oracle(b, window=1000, landmark_chunk=0)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_block_mask_special_cases():
    rng = np.random.default_rng(12)
    b = W.build_batch(rng, name="m", kind="bf16", Hq=2, Hkv=1, d=32, page_size=64,
                      ctx=[384], q_len=[384], keep_dense=True)
    O, L = run_oracle(b)
    ones = np.ones((1, 1, 3, 3), dtype=np.uint8)
    O1, L1 = run_oracle(b, block_mask=ones)
    assert np.array_equal(O, O1) and np.array_equal(L, L1)
    # diagonal-only mask == independent causal attention inside each 128-token block
    diag = np.eye(3, dtype=np.uint8)[None, None]
    Od, _ = run_oracle(b, block_mask=diag)
    q = torch.from_numpy(dequant64(b.q))
    k = torch.from_numpy(dequant64(b.dense_k[0]))
    v = torch.from_numpy(dequant64(b.dense_v[0]))
    for blk in range(3):
        sl = slice(128 * blk, 128 * (blk + 1))
        for h in range(2):
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[sl, h][None], k[sl, 0][None], v[sl, 0][None], is_causal=True, scale=b.softmax_scale)[0]
            assert float((ref - torch.from_numpy(Od[sl, h])).abs().max()) <= 1e-12


def test_expand_to_chunk_changes_only_unaligned_rows():
    rng = np.random.default_rng(13)
    W_, C = 96, 32
    b = W.build_batch(rng, name="w", kind="bf16", Hq=2, Hkv=1, d=32, page_size=64,
                      ctx=[300], q_len=[300], identity_pages=True, window=W_, landmark_chunk=C)
    Oe, Le = run_oracle(b, window_expand_to_chunk=True)
    On, Ln = run_oracle(b, window_expand_to_chunk=False)
    pos = np.arange(300)
    same = (pos - W_ + 1 <= 0) | ((pos - W_ + 1) % C == 0)
    assert np.array_equal(Oe[same], On[same]) and np.array_equal(Le[same], Ln[same])
    assert np.all(np.abs(Le[~same] - Ln[~same]).max(axis=1) > 0)


def _empty_row_batch():
    """A chunk where every other row sees no key although the key span of its
    row block is non-empty: window 1 (no expansion) leaves each query only its
    own key, and landmark chunk 2 hides the keys j with (j + 1) even, so a
    query at an odd position sees nothing."""
    rng = np.random.default_rng(47)
    return W.build_batch(rng, name="empty_rows", kind="f32", Hq=4, Hkv=2, d=16, page_size=16,
                         ctx=[23, 9], q_len=[13, 9], keep_dense=True, window=1,
                         window_expand_to_chunk=False, landmark_chunk=2)


def test_rows_without_visible_keys_inside_a_nonempty_span():
    b = _empty_row_batch()
    O, L = run_oracle(b)
    Ob, Lb = _brute(b)
    qsl, ctx = b.query_start_loc.tolist(), b.seq_lens.tolist()
    empty = np.zeros(b.total_q, dtype=bool)
    for s in range(b.num_seqs):
        for t in range(qsl[s], qsl[s + 1]):
            pos = ctx[s] - (qsl[s + 1] - qsl[s]) + (t - qsl[s])
            empty[t] = pos % 2 == 1
    assert empty.any() and (~empty).any()
    # brute force and the definition: O = 0 and LSE = -inf exactly, no NaN
    assert np.all(Ob[empty] == 0.0) and np.all(Lb[empty] == -math.inf)
    assert not np.isnan(O).any() and not np.isnan(L).any()
    assert np.all(O[empty] == 0.0) and np.all(L[empty] == -math.inf)
    # the other rows see exactly one key: O = that value row, LSE = its score
    assert np.abs(O[~empty] - Ob[~empty]).max() <= 1e-12
    assert np.abs(L[~empty] - Lb[~empty]).max() <= 1e-12
