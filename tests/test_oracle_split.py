"""Pins for oracle.split: the LSE-weighted combine equals unsplit attention."""
import math

import numpy as np

from attention_paged_kv_attn_amd import workloads as W
from oracle.split import combine, merge_raw_base2, split_paged_attention
from tests.oracle_helpers import oracle_scales, run_oracle, stored_np


def _args(b):
    return (stored_np(b.q, b.kind), stored_np(b.k_cache, b.kind), stored_np(b.v_cache, b.kind),
            b.block_table.numpy(), b.seq_lens.numpy(), b.query_start_loc.numpy())


def _kw(b):
    return dict(kind=b.kind, softmax_scale=b.softmax_scale, kv_layout=b.kv_layout, causal=b.causal,
                window=b.window, window_expand_to_chunk=b.window_expand_to_chunk,
                landmark_chunk=b.landmark_chunk, scales=oracle_scales(b))


def test_any_partition_combines_to_unsplit():
    rng = np.random.default_rng(5)
    for b in (W.tiny_hybrid(), W.splitk_decode(q_len=4, batch=5, ctx_lo=64, ctx_hi=700)):
        O, L = run_oracle(b)
        cuts = []
        for ctx in b.seq_lens.tolist():
            k = int(rng.integers(1, 5))
            cuts.append(sorted(set(int(x) for x in rng.integers(1, ctx, size=k))))
        Os, Ls = split_paged_attention(*_args(b), boundaries=cuts, **_kw(b))
        assert np.abs(Os - O).max() <= 1e-12
        assert np.abs(Ls - L).max() <= 1e-12


def test_empty_part_is_exact_noop():
    b = W.tiny_hybrid()
    O, L = run_oracle(b)
    ctx = b.seq_lens.tolist()
    # first part empty ([0,0)), second part is everything
    Os, Ls = split_paged_attention(*_args(b), boundaries=[[0] for _ in ctx], **_kw(b))
    assert np.array_equal(Os, O) and np.array_equal(Ls, L)


def test_all_empty_rows():
    O, L = combine(np.full((3, 2), -math.inf), np.zeros((3, 2, 4)))
    assert np.all(O == 0) and np.all(L == -math.inf)


def test_raw_base2_merge_matches_combine():
    rng = np.random.default_rng(1)
    d = 8
    s0 = rng.standard_normal(10)
    s1 = rng.standard_normal(7) + 3
    v0 = rng.standard_normal((10, d))
    v1 = rng.standard_normal((7, d))
    ln2 = math.log(2)

    def raw(s, v):                       # base-2 raw state of one chunk
        s2 = s / ln2
        m = s2.max()
        w = 2.0 ** (s2 - m)
        return m, w.sum(), w @ v

    m, l, o = merge_raw_base2(*raw(s0, v0), *raw(s1, v1))
    lse_merged = (m + math.log2(l)) * ln2
    out_merged = o / l
    # direct, unsplit
    s = np.concatenate([s0, s1])
    v = np.concatenate([v0, v1])
    p = np.exp(s - s.max())
    assert abs(lse_merged - (s.max() + math.log(p.sum()))) <= 1e-12
    assert np.abs(out_merged - (p @ v) / p.sum()).max() <= 1e-12
    # and the normalised-partial combine agrees
    parts_l = np.array([[s0.max() + math.log(np.exp(s0 - s0.max()).sum())],
                        [s1.max() + math.log(np.exp(s1 - s1.max()).sum())]])
    parts_o = np.array([[(np.exp(s0 - s0.max()) @ v0) / np.exp(s0 - s0.max()).sum()],
                        [(np.exp(s1 - s1.max()) @ v1) / np.exp(s1 - s1.max()).sum()]])
    Oc, Lc = combine(parts_l, parts_o)
    assert np.abs(Oc[0] - out_merged).max() <= 1e-12 and abs(Lc[0] - lse_merged) <= 1e-12
