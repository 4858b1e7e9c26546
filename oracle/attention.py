"""The definition of paged-KV attention forward — oracle side, test infrastructure.

Parity status: pinned (tests/test_oracle_attention.py: brute force on dense
inputs, torch scaled_dot_product_attention in float64, closed forms with
Q = 0, one-hot V, constant V, single visible key, the LSE identity, page
permutation invariance, NHD == HND, GQA replication, window/landmark and
block-mask special cases).

What is computed, for every sequence b, query token i and query head h:

* paging ("Triton-TLE rewrite of Tencent HPC-Ops Attention", §1.2 and §3.2):
  key j of sequence b lives in physical page block_table[b, j // page_size]
  at slot j % page_size; the cache is addressed by the logical coordinates
  (page, slot, kv_head, dim) and the NHD / HND layouts differ only in the
  order of slot and kv_head.
* GQA ("vLLM Triton Attention Backend Deep Dive", §3 Q blocks): query head h
  reads kv head g = h // (Hq / Hkv).
* positions: seq_lens[b] counts every key of the sequence including the
  q_len new tokens, so query token i sits at pos = seq_len - q_len + i
  ("Chunked Prefill ... Triton hybrid attention": a decode row reads its whole
  history, a chunk is causal within itself and sees its history unmasked).
* visibility: j < seq_len, and j <= pos when causal, and the sliding window
  j >= left(pos) with left rounded down to a multiple of the landmark chunk C
  when expand_to_chunk is set, and (j + 1) mod C != 0 for landmark masking
  ("HiLS-Attention sliding-window forward", §3 stage 1), and the 128x128
  block-mask tile (pos // tile, j // tile) set to 1 ("Triton-TLE ... HPC-Ops",
  §1.2, block-sparse prefill only processes valid KV tiles).
* s_j = scale * <q_hat, k_hat_j>; O = sum_j softmax(s)_j v_hat_j over the
  visible keys; LSE = ln sum_j exp(s_j) (natural log, "HiLS-Attention", §3
  stage 1).  A row with no visible key has O = 0 and LSE = -inf.
* stored values are upcast exactly: f32 as is, bf16 by widening its bits,
  e4m3 through the E4M3FN table times its scale (per tensor, or per
  (physical page, kv head) for K and V; Q per tensor, or per (query token,
  query head) as in the FP8 decode quantisation path of "Triton-TLE rewrite
  of Tencent HPC-Ops Attention", §3 Dynamic Decode, its FP8 results).  The fp32 softmax scale is used as
  passed, widened to float64.

Everything is float64.  Query rows are processed in blocks of row_block
tokens only to cap memory; within a block the key columns are restricted to
the span that holds every visible key of the block (masked keys contribute
an exact zero, so this changes no value).
"""
import math
import numpy as np

from . import fp8

KINDS = ("f32", "bf16", "e4m3")


def upcast(stored, kind: str) -> np.ndarray:
    """Exact widening of stored element values to float64."""
    if kind == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if kind == "bf16":
        bits = np.asarray(stored)
        if bits.dtype != np.uint16:
            raise TypeError("bf16 values must be passed as their uint16 bit patterns")
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if kind == "e4m3":
        return fp8.decode(stored)
    raise ValueError(f"unknown element kind {kind!r}")


def window_left(pos: np.ndarray, window: int, expand_to_chunk: bool, chunk: int) -> np.ndarray:
    """First key a query at `pos` may see under a sliding window of `window` keys."""
    left = np.maximum(0, pos - window + 1)
    if expand_to_chunk and chunk > 0:
        left = (left // chunk) * chunk
    return left


def visible(pos: np.ndarray, keys: np.ndarray, ctx: int, *, causal: bool, window: int,
            expand_to_chunk: bool, landmark_chunk: int, mask_rows=None, mask_tile: int = 128) -> np.ndarray:
    """Boolean [len(pos), len(keys)]: may the query at pos[r] attend to key keys[c]?

    mask_rows, when given, is the uint8 block-mask slab [n_q_tiles, n_k_tiles]
    of this sequence and query head.
    """
    pos = np.asarray(pos, dtype=np.int64)[:, None]
    j = np.asarray(keys, dtype=np.int64)[None, :]
    vis = j < ctx
    if causal:
        vis = vis & (j <= pos)
    if window > 0:
        vis = vis & (j >= window_left(pos, window, expand_to_chunk, landmark_chunk))
    if landmark_chunk > 0:
        vis = vis & ((j + 1) % landmark_chunk != 0)
    if mask_rows is not None:
        mask_rows = np.asarray(mask_rows)
        vis = vis & (mask_rows[pos // mask_tile, j // mask_tile] != 0)
    return vis


def _gather(cache, kind, pages, slots, g, kv_layout):
    if kv_layout == "NHD":       # [num_pages, page_size, Hkv, d]
        raw = cache[pages, slots, g, :]
    elif kv_layout == "HND":     # [num_pages, Hkv, page_size, d]
        raw = cache[pages, g, slots, :]
    else:
        raise ValueError(kv_layout)
    return upcast(raw, kind)


def paged_attention(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, *,
                    kind: str, softmax_scale, kv_layout: str = "NHD", causal: bool = True,
                    window: int = 0, window_expand_to_chunk: bool = True, landmark_chunk: int = 0,
                    block_mask=None, block_mask_tile: int = 128, scales=None,
                    key_range=None, row_block: int = 1024, rows=None):
    """O [total_q, Hq, d] and LSE [total_q, Hq], both float64.

    q        stored values [total_q, Hq, d]
    k_cache  stored values, [num_pages, page_size, Hkv, d] (NHD) or
             [num_pages, Hkv, page_size, d] (HND); v_cache likewise
    block_table int [B, max_pages]; seq_lens int [B]; query_start_loc int [B+1]
    block_mask  uint8 [B, H_m, n_q_tiles, n_k_tiles] with H_m in {1, Hq}, or None
    scales   for kind "e4m3": {"mode": "tensor"|"page_head", "q": float,
             "k": float or [num_pages, Hkv], "v": same}, and optionally
             "q_mode": "token_head" with "q" a [total_q, Hq] array
    key_range   optional int [B, 2]: only keys lo <= j < hi count (split reference)
    rows     optional boolean [total_q]: compute only these query rows
             (others are left as NaN) — used to evaluate sampled outputs.
    """
    q = np.asarray(q)
    total_q, Hq, d = q.shape
    Hkv = k_cache.shape[2] if kv_layout == "NHD" else k_cache.shape[1]
    page_size = k_cache.shape[1] if kv_layout == "NHD" else k_cache.shape[2]
    num_pages = k_cache.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    block_table = np.asarray(block_table, dtype=np.int64)
    B = seq_lens.shape[0]
    if qsl.shape[0] != B + 1 or qsl[0] != 0 or qsl[-1] != total_q:
        raise ValueError("query_start_loc must be a [B+1] prefix ending at total_q")
    sigma = float(np.float32(softmax_scale))

    if kind == "e4m3":
        if scales is None:
            raise ValueError("e4m3 inputs need scales")
        q_scale = _q_scale(scales, total_q, Hq)
    else:
        q_scale = None

    O = np.full((total_q, Hq, d), np.nan)
    LSE = np.full((total_q, Hq), np.nan)

    for b in range(B):
        q0, q1 = int(qsl[b]), int(qsl[b + 1])
        ql, ctx = q1 - q0, int(seq_lens[b])
        if ql < 0 or ql > ctx:
            raise ValueError(f"sequence {b}: need 0 <= q_len <= seq_len")
        if ql == 0:
            continue
        n_pages_b = -(-ctx // page_size)
        pages_b = block_table[b, :n_pages_b]
        if np.any(pages_b < 0) or np.any(pages_b >= num_pages):
            raise ValueError(f"sequence {b}: block_table entry out of range")
        key_lo, key_hi = (0, ctx) if key_range is None else (int(key_range[b][0]), int(key_range[b][1]))
        tok = np.arange(q0, q1)
        if rows is not None:
            tok = tok[np.asarray(rows)[q0:q1]]
            if tok.size == 0:
                continue
        for g in range(Hkv):
            for ib in range(0, tok.size, row_block):
                t = tok[ib:ib + row_block]
                pos = ctx - ql + (t - q0)
                # span of keys any row of this block can see
                hi = min(ctx, key_hi, int(pos.max()) + 1 if causal else ctx)
                lo = max(key_lo, int(window_left(pos, window, window_expand_to_chunk,
                                                 landmark_chunk).min()) if window > 0 else 0)
                qhat = upcast(q[t, g * G:(g + 1) * G, :], kind)                # [n, G, d]
                if q_scale is not None:
                    qhat = qhat * (q_scale if np.isscalar(q_scale)
                                   else q_scale[t, g * G:(g + 1) * G, None])
                if hi <= lo:
                    O[t, g * G:(g + 1) * G, :] = 0.0
                    LSE[t, g * G:(g + 1) * G] = -math.inf
                    continue
                j = np.arange(lo, hi)
                pages, slots = pages_b[j // page_size], j % page_size
                khat = _gather(k_cache, kind, pages, slots, g, kv_layout)
                vhat = _gather(v_cache, kind, pages, slots, g, kv_layout)
                if kind == "e4m3":
                    khat = khat * _kv_scale(scales, "k", pages, g)
                    vhat = vhat * _kv_scale(scales, "v", pages, g)
                for hi_ in range(G):
                    h = g * G + hi_
                    mask_rows = None
                    if block_mask is not None:
                        hm = 0 if block_mask.shape[1] == 1 else h
                        mask_rows = block_mask[b, hm]
                    vis = visible(pos, j, ctx, causal=causal, window=window,
                                  expand_to_chunk=window_expand_to_chunk,
                                  landmark_chunk=landmark_chunk, mask_rows=mask_rows,
                                  mask_tile=block_mask_tile)
                    s = (qhat[:, hi_, :] @ khat.T) * sigma
                    o, lse = _softmax_rows(s, vis, vhat)
                    O[t, h, :] = o
                    LSE[t, h] = lse
    return O, LSE


def _q_scale(scales, total_q, Hq):
    """The Q dequantisation scale: one float, or per (query token, query head)."""
    mode = scales.get("q_mode", "tensor")
    if mode == "tensor":
        return float(np.float32(scales["q"]))
    if mode == "token_head":
        s = np.asarray(scales["q"], dtype=np.float32).astype(np.float64)
        if s.shape != (total_q, Hq):
            raise ValueError("per-(token, head) Q scales must be [total_q, Hq]")
        return s
    raise ValueError(mode)


def _kv_scale(scales, which, pages, g):
    s = scales[which]
    if scales["mode"] == "tensor":
        return float(np.float32(s))
    if scales["mode"] == "page_head":
        return np.asarray(s, dtype=np.float32).astype(np.float64)[pages, g][:, None]
    raise ValueError(scales["mode"])


def _softmax_rows(s, vis, vhat):
    """Masked softmax of score rows s [n, m] against values vhat [m, d]."""
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])           # exp(-inf) = 0 exactly on masked keys
    z = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (e @ vhat) / z[:, None]
        lse = m_safe + np.log(z)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse
