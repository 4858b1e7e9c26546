"""Host logic of the benchmark that its roofline figures rest on, checked on
the CPU: the visible (row, key) pairs that price a run's flops (4 d per pair)
and the keys per kv head that price its bytes, against a brute-force count of
the oracle's own visibility rule on small batches."""
import zlib

import numpy as np
import pytest

import bench
from attention_paged_kv_attn_amd import workloads as W
from oracle.attention import visible


def _brute(batch):
    ctx = batch.seq_lens.numpy().astype(np.int64)
    qsl = batch.query_start_loc.numpy().astype(np.int64)
    bm = None if batch.block_mask is None else batch.block_mask.numpy()
    pairs = 0
    keys = 0
    for b in range(len(ctx)):
        ql = int(qsl[b + 1] - qsl[b])
        if ql == 0:
            continue
        pos = ctx[b] - ql + np.arange(ql)
        vis = visible(pos, np.arange(ctx[b]), int(ctx[b]), causal=batch.causal, window=batch.window,
                      expand_to_chunk=batch.window_expand_to_chunk, landmark_chunk=batch.landmark_chunk,
                      mask_rows=None if bm is None else bm[b, 0], mask_tile=batch.block_mask_tile)
        vis = np.broadcast_to(vis, (ql, int(ctx[b])))    # (one row of keys when no rule depends on pos)
        pairs += int(vis.sum())
        keys += int(vis.any(axis=0).sum())
    return pairs * batch.num_q_heads, keys


CASES = {
    "decode_mtp": dict(Hq=8, Hkv=2, ctx=[37, 300, 129, 64], q_len=[1, 4, 2, 3]),
    "prefill_chunks": dict(Hq=8, Hkv=2, ctx=[300, 250, 90], q_len=[300, 100, 17]),
    "noncausal": dict(Hq=4, Hkv=1, ctx=[200, 75], q_len=[5, 75], causal=False),
    "window": dict(Hq=4, Hkv=1, ctx=[500, 333], q_len=[200, 1], window=96, window_expand_to_chunk=False),
    "window_landmarks": dict(Hq=4, Hkv=1, ctx=[500, 333, 64], q_len=[200, 3, 64], window=96, landmark_chunk=16),
    "landmarks_only": dict(Hq=4, Hkv=1, ctx=[300, 129], q_len=[300, 1], landmark_chunk=64),
    "block_mask": dict(Hq=8, Hkv=2, ctx=[600, 520], q_len=[600, 520], block_mask_skip=0.6, block_mask_tile=128),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_visible_pairs_and_keys_match_brute_force(name):
    kw = dict(CASES[name])
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    b = W.build_batch(rng, name=name, kind="bf16", d=64, page_size=16, poison=False, **kw)
    pairs, keys = bench.visible_pairs_and_keys(b)
    bp, bk = _brute(b)
    assert pairs == bp
    assert keys == bk
