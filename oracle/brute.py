"""Brute-force attention with pure-Python loops — oracle side, test infrastructure.

Parity status: this module is itself a pin for oracle.attention.  It works on
dense (unpaged) per-sequence K/V, re-states the visibility rule with plain
if-statements and sums with math.exp, so it shares neither the gather, the
vectorised mask nor the NumPy softmax with oracle.attention.  Use on tiny
inputs only.

Rule sources: causal within a chunk and full history for decode rows
("Chunked Prefill ... Triton hybrid attention", mask specialisation);
sliding window, expand_to_chunk and landmark masking ("HiLS-Attention
sliding-window forward", §3 stage 1); block-mask tiles ("Triton-TLE rewrite of
Tencent HPC-Ops Attention", §1.2).
"""
import math


def is_visible(pos, j, ctx, *, causal=True, window=0, expand_to_chunk=True, chunk=0,
               mask=None, tile=128):
    if j < 0 or j >= ctx:
        return False
    if causal and j > pos:
        return False
    if window > 0:
        left = pos - window + 1
        if left < 0:
            left = 0
        if expand_to_chunk and chunk > 0:
            left = left - (left % chunk)
        if j < left:
            return False
    if chunk > 0 and (j + 1) % chunk == 0:
        return False
    if mask is not None and not mask[pos // tile][j // tile]:
        return False
    return True


def attend_row(qvec, keys, values, scale, vis):
    """One query row.  qvec: list[d]; keys/values: list of list[d]; vis: list[bool]."""
    scores = []
    for j, k in enumerate(keys):
        if vis[j]:
            acc = 0.0
            for a, b in zip(qvec, k):
                acc += a * b
            scores.append((j, acc * scale))
    if not scores:
        return [0.0] * len(qvec), -math.inf
    m = max(s for _, s in scores)
    z = 0.0
    out = [0.0] * len(qvec)
    for j, s in scores:
        w = math.exp(s - m)
        z += w
        for c, v in enumerate(values[j]):
            out[c] += w * v
    return [o / z for o in out], m + math.log(z)


def attention_batch(q_rows, dense_k, dense_v, seq_lens, query_start_loc, *, Hq, scale,
                    causal=True, window=0, expand_to_chunk=True, chunk=0, block_mask=None, tile=128):
    """q_rows: nested lists [total_q][Hq][d] (float); dense_k[b]: [ctx_b][Hkv][d].

    Returns (O nested [total_q][Hq][d], LSE [total_q][Hq]).
    """
    Hkv = len(dense_k[0][0])
    G = Hq // Hkv
    O, L = [], []
    for b in range(len(seq_lens)):
        ctx = seq_lens[b]
        q0, q1 = query_start_loc[b], query_start_loc[b + 1]
        ql = q1 - q0
        for t in range(q0, q1):
            pos = ctx - ql + (t - q0)
            o_row, l_row = [], []
            for h in range(Hq):
                g = h // G
                mask = None
                if block_mask is not None:
                    mask = block_mask[b][0 if len(block_mask[b]) == 1 else h]
                vis = [is_visible(pos, j, ctx, causal=causal, window=window,
                                  expand_to_chunk=expand_to_chunk, chunk=chunk, mask=mask, tile=tile)
                       for j in range(ctx)]
                keys = [dense_k[b][j][g] for j in range(ctx)]
                vals = [dense_v[b][j][g] for j in range(ctx)]
                o, lse = attend_row(q_rows[t][h], keys, vals, scale, vis)
                o_row.append(o)
                l_row.append(lse)
            O.append(o_row)
            L.append(l_row)
    return O, L
