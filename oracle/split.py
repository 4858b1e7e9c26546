"""Split-K reference: attention over a key range and the LSE-weighted combine.

Oracle side, test infrastructure.  Parity status: pinned
(tests/test_oracle_split.py: any partition of the keys combines to the
unsplit result; empty parts are exact no-ops; the two-state merge of raw
online-softmax states gives the same result).

* "Triton-TLE rewrite of Tencent HPC-Ops Attention", §1.2 (dynamic decode):
  the Split-K stage emits a local output and LSE per KV chunk and the Combine
  stage re-normalises the chunk outputs by their LSE, which is mathematically
  the same as full attention.
* same page, §3.3: two raw online-softmax states (m_i, l_i, o_i) in base 2
  merge as m = max(m_0, m_1), w_i = 2^(m_i - m), l = sum l_i w_i,
  o = sum o_i w_i, normalised only at the end.
"""
import math
import numpy as np

from .attention import paged_attention


def combine(lse_parts, o_parts):
    """lse_parts [S, rows], o_parts [S, rows, d] (normalised partial outputs).

    Returns O [rows, d], LSE [rows]: M = max_s LSE_s, LSE = M + ln sum_s
    exp(LSE_s - M), O = sum_s exp(LSE_s - LSE) O_s.  Parts with LSE = -inf
    weigh 0; if every part is -inf the row is O = 0, LSE = -inf.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    empty = ~np.isfinite(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.exp(lse_parts - M_safe[None, :])
    lse = M_safe + np.log(np.where(empty, 1.0, w.sum(axis=0)))
    coef = np.exp(lse_parts - lse[None, :])
    o_parts = np.where(np.isfinite(lse_parts)[:, :, None], o_parts, 0.0)
    O = (coef[:, :, None] * o_parts).sum(axis=0)
    O[empty] = 0.0
    lse[empty] = -math.inf
    return O, lse


def merge_raw_base2(m0, l0, o0, m1, l1, o1):
    """Merge two unnormalised base-2 online-softmax states (m, l, o)."""
    m = max(m0, m1)
    if m == -math.inf:
        return m, 0.0, np.zeros_like(np.asarray(o0, dtype=np.float64))
    w0 = 2.0 ** (m0 - m)
    w1 = 2.0 ** (m1 - m)
    return m, l0 * w0 + l1 * w1, np.asarray(o0) * w0 + np.asarray(o1) * w1


def split_paged_attention(*args, boundaries, **kw):
    """Attention with the keys of sequence b cut at boundaries[b] (sorted
    interior cut points), each part computed alone and then combined."""
    seq_lens = np.asarray(args[4])
    B = seq_lens.shape[0]
    n_parts = max(len(c) for c in boundaries) + 1
    lses, outs = [], []
    for p in range(n_parts):
        kr = np.zeros((B, 2), dtype=np.int64)
        for b in range(B):
            cuts = [0] + list(boundaries[b]) + [int(seq_lens[b])]
            if p + 1 < len(cuts):
                kr[b] = (cuts[p], cuts[p + 1])
            else:
                kr[b] = (0, 0)               # this sequence has fewer parts: empty range
        o, l = paged_attention(*args, key_range=kr, **kw)
        outs.append(o)
        lses.append(l)
    total_q, Hq, d = outs[0].shape
    O, L = combine(np.stack(lses).reshape(n_parts, -1),
                   np.stack(outs).reshape(n_parts, -1, d))
    return O.reshape(total_q, Hq, d), L.reshape(total_q, Hq)
