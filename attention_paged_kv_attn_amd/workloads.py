"""Seeded synthetic inputs shaped like the workloads on the paged-attention pages.

This module only draws and lays out inputs: random values, sequence lengths,
page permutations, block tables, block masks and FP8 scales.  It holds none of
the attention arithmetic, imports neither the oracle nor the HIP binding, and
is the one piece shared by the tests, the benchmark and the oracle checks.

Recipe (common to all workloads)
* One ``numpy.random.default_rng(seed)`` stream, drawn in the order
  lengths -> page permutation -> value seeds -> block mask.  The N(0, 1)
  float32 values come from three ``torch.Generator`` streams seeded from it,
  one each for Q, K and V (K and V drawn sequence by sequence).  (The MTP decode runs seed Q from
  a second numpy stream seeded 200 + q_len so that the K/V of one batch are
  shared by every q_len.)
* Values are rounded to the stored type by torch's round-to-nearest-even
  casts.  FP8 (E4M3FN) values are divided by a scale
  amax / 448 first (1.0 when amax is 0): one scale per tensor, or for K and V
  one per (physical page, kv head).
* The physical page pool holds exactly the pages the batch needs unless a
  larger pool is asked for; the block table is a random permutation of the
  pool cut per sequence in batch order (identity when asked), padded with -1.
* Cache slots past a sequence's end and unused pages are filled with NaN
  (0x7F for FP8) for correctness runs (poison=True) and with zeros otherwise.
* seq_lens[b] counts every key of sequence b including its q_len new tokens.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

F8_MAX = 448.0
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}


@dataclass
class PagedBatch:
    name: str
    kind: str                     # stored element type of Q/K/V: "f32" | "bf16" | "e4m3"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_layout: str                # "NHD": [pages, page_size, Hkv, d]; "HND": [pages, Hkv, page_size, d]
    q: torch.Tensor               # [total_q, Hq, d]
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor     # int32 [B, max_pages], -1 padded
    seq_lens: torch.Tensor        # int32 [B]
    query_start_loc: torch.Tensor  # int32 [B + 1]
    softmax_scale: float          # an fp32 value
    causal: bool = True
    window: int = 0
    window_expand_to_chunk: bool = True
    landmark_chunk: int = 0
    block_mask: Optional[torch.Tensor] = None   # uint8 [B, H_m, n_q_tiles, n_k_tiles]
    block_mask_tile: int = 128
    scales: Optional[dict] = None  # {"mode": "tensor"|"page_head", "q": f32[1], "k": f32[1] or [pages, Hkv], "v": ...}
    out_heads_major: bool = False  # outputs laid out (B, Hq, Lq, d) / (B, Hq, Lq) instead of token-major
    dense_k: Optional[list] = None  # per sequence [ctx, Hkv, d] stored values (tiny workloads only)
    dense_v: Optional[list] = None
    info: dict = field(default_factory=dict)
    max_q_len: int = 0            # the largest q_len of the batch (0 = not stated)
    min_q_len: int = 0            # the smallest non-zero q_len of the batch (0 = not stated)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    def to(self, device) -> "PagedBatch":
        """Copy every tensor to `device` (dense copies stay on the host)."""
        kw = dict(self.__dict__)
        for key in ("q", "k_cache", "v_cache", "block_table", "seq_lens", "query_start_loc", "block_mask"):
            if kw[key] is not None:
                kw[key] = kw[key].to(device)
        if self.scales is not None:
            kw["scales"] = {k: (v.to(device) if isinstance(v, torch.Tensor) else v)
                            for k, v in self.scales.items()}
        return PagedBatch(**kw)


def _cast(x32: np.ndarray, kind: str, scale: float = 1.0) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x32))
    if kind == "e4m3":
        t = t / torch.tensor(scale, dtype=torch.float32)
    return t.to(TORCH_DTYPE[kind])


def _f8_scale(amax: float) -> float:
    return float(np.float32(amax / F8_MAX)) if amax > 0 else 1.0


def _poison_fill(shape, kind, poison):
    dt = TORCH_DTYPE[kind]
    if not poison:
        return torch.zeros(shape, dtype=dt)
    if kind == "e4m3":
        return torch.full(shape, 0x7F, dtype=torch.uint8).view(dt)
    return torch.full(shape, float("nan"), dtype=dt)


def build_batch(rng: np.random.Generator, *, name: str, kind: str, Hq: int, Hkv: int, d: int,
                page_size: int, ctx, q_len, kv_layout: str = "NHD", num_pages: Optional[int] = None,
                q_rng: Optional[np.random.Generator] = None, q_gain: float = 1.0,
                identity_pages: bool = False, poison: bool = True, keep_dense: bool = False,
                quant_mode: Optional[str] = None, q_quant: str = "tensor",
                softmax_scale: Optional[float] = None, causal: bool = True, window: int = 0, window_expand_to_chunk: bool = True,
                landmark_chunk: int = 0, block_mask_skip: Optional[float] = None,
                block_mask_tile: int = 128, out_heads_major: bool = False) -> PagedBatch:
    """Lay out one batch.  `ctx` and `q_len` (per sequence) must already be drawn."""
    ctx = [int(c) for c in ctx]
    q_len = [int(x) for x in q_len]
    B = len(ctx)
    assert all(0 <= ql <= c for ql, c in zip(q_len, ctx)), "need q_len <= seq_len"
    n_pages_seq = [-(-c // page_size) for c in ctx]
    need = sum(n_pages_seq)
    num_pages = need if num_pages is None else int(num_pages)
    assert num_pages >= need
    max_pages = max(1, max(n_pages_seq))

    # page permutation -> block table
    perm = np.arange(num_pages) if identity_pages else rng.permutation(num_pages)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :n_pages_seq[b]] = perm[off:off + n_pages_seq[b]]
        off += n_pages_seq[b]

    # value streams
    q_seed = int((q_rng or rng).integers(0, 2 ** 62))
    k_seed = int(rng.integers(0, 2 ** 62))
    v_seed = int(rng.integers(0, 2 ** 62))
    total_q = sum(q_len)
    qs = torch.randn((total_q, Hq, d), generator=torch.Generator().manual_seed(q_seed)).numpy()
    if q_gain != 1.0:
        qs = qs * np.float32(q_gain)
    k_gen = torch.Generator().manual_seed(k_seed)
    v_gen = torch.Generator().manual_seed(v_seed)

    scales = None
    ks = vs = None
    if kind == "e4m3":
        if quant_mode not in ("tensor", "page_head"):
            raise ValueError("e4m3 needs quant_mode 'tensor' or 'page_head'")
        # scales need every value first: draw all K, then all V
        ks = [torch.randn((c, Hkv, d), generator=k_gen).numpy() for c in ctx]
        vs = [torch.randn((c, Hkv, d), generator=v_gen).numpy() for c in ctx]
        if q_quant == "tensor":
            q_s = np.float32(_f8_scale(float(np.abs(qs).max()) if qs.size else 0.0))
        elif q_quant == "token_head":
            # one scale per (query token, query head): its own amax over d
            amax = np.abs(qs).max(axis=2) if qs.size else np.zeros(qs.shape[:2], np.float32)
            q_s = np.vectorize(lambda a: _f8_scale(float(a)), otypes=[np.float32])(amax)
            q_s = q_s.reshape(qs.shape[:2]).astype(np.float32)
        else:
            raise ValueError("q_quant must be 'tensor' or 'token_head'")
        if quant_mode == "tensor":
            k_s = _f8_scale(max((float(np.abs(k).max()) for k in ks if k.size), default=0.0))
            v_s = _f8_scale(max((float(np.abs(v).max()) for v in vs if v.size), default=0.0))
            k_sc = np.float32(k_s)
            v_sc = np.float32(v_s)
        else:
            k_sc = np.ones((num_pages, Hkv), dtype=np.float32)
            v_sc = np.ones((num_pages, Hkv), dtype=np.float32)
            for b in range(B):
                for p in range(n_pages_seq[b]):
                    sl = slice(p * page_size, min((p + 1) * page_size, ctx[b]))
                    for arr, sc in ((ks[b], k_sc), (vs[b], v_sc)):
                        amax = np.abs(arr[sl]).max(axis=(0, 2))
                        sc[bt[b, p]] = [_f8_scale(float(a)) for a in amax]
        scales = {"mode": quant_mode, "q_mode": q_quant,
                  "q": torch.from_numpy(np.atleast_1d(q_s).astype(np.float32).copy()),
                  "k": torch.from_numpy(np.atleast_1d(k_sc).astype(np.float32).copy()),
                  "v": torch.from_numpy(np.atleast_1d(v_sc).astype(np.float32).copy())}
        if q_quant == "tensor":
            q_t = _cast(qs, kind, float(q_s))
        else:
            q_t = _cast(qs / q_s[:, :, None], kind)
    else:
        q_t = _cast(qs, kind)

    shape = (num_pages, page_size, Hkv, d) if kv_layout == "NHD" else (num_pages, Hkv, page_size, d)
    dt = TORCH_DTYPE[kind]
    k_cache = torch.empty(shape, dtype=dt)
    v_cache = torch.empty(shape, dtype=dt)
    used = np.zeros(num_pages, dtype=bool)
    dense_k, dense_v = ([], []) if keep_dense else (None, None)
    for b in range(B):
        npg = n_pages_seq[b]
        kb = ks[b] if ks is not None else torch.randn((ctx[b], Hkv, d), generator=k_gen).numpy()
        vb = vs[b] if vs is not None else torch.randn((ctx[b], Hkv, d), generator=v_gen).numpy()
        if npg == 0:
            if dense_k is not None:
                dense_k.append(_cast(kb, kind) if kind != "e4m3" else torch.empty((0, Hkv, d), dtype=dt))
                dense_v.append(_cast(vb, kind) if kind != "e4m3" else torch.empty((0, Hkv, d), dtype=dt))
            continue
        used[bt[b, :npg]] = True
        pages = torch.from_numpy(bt[b, :npg].astype(np.int64))
        for arr, cache, dense, which in ((kb, k_cache, dense_k, "k"), (vb, v_cache, dense_v, "v")):
            if kind == "e4m3":
                if quant_mode == "tensor":
                    stored = _cast(arr, kind, float(scales[which][0]))
                else:
                    sc = scales[which].numpy()
                    per_tok = np.repeat(sc[bt[b, :npg]], page_size, axis=0)[:ctx[b]]   # [ctx, Hkv]
                    stored = _cast(arr / per_tok[:, :, None], kind)
            else:
                stored = _cast(arr, kind)
            if dense is not None:
                dense.append(stored.clone())
            padded = _poison_fill((npg * page_size, Hkv, d), kind, poison)
            padded[:ctx[b]] = stored
            padded = padded.view(npg, page_size, Hkv, d)
            if kv_layout == "HND":
                padded = padded.transpose(1, 2)
            cache[pages] = padded
        del kb, vb
    free = torch.from_numpy(np.nonzero(~used)[0])
    if free.numel():
        fill = _poison_fill((free.numel(),) + shape[1:], kind, poison)
        k_cache[free] = fill
        v_cache[free] = fill
    del ks, vs

    block_mask = None
    info = {}
    if block_mask_skip is not None:
        nqt = -(-max(ctx) // block_mask_tile)
        keep = rng.random((B, 1, nqt, nqt)) >= block_mask_skip
        keep[:, :, np.arange(nqt), np.arange(nqt)] = True          # diagonal tiles always kept
        block_mask = torch.from_numpy(keep.astype(np.uint8))
        tri = np.tril(np.ones((nqt, nqt), dtype=bool))
        causal_tiles = int(tri.sum()) * B
        kept = int((keep[:, 0] & tri[None]).sum())
        info["tile_skip_ratio"] = 1.0 - kept / causal_tiles

    qsl = np.zeros(B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_len)
    if softmax_scale is None:
        softmax_scale = float(np.float32(1.0 / math.sqrt(d)))
    return PagedBatch(name=name, kind=kind, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                      page_size=page_size, kv_layout=kv_layout, q=q_t, k_cache=k_cache,
                      v_cache=v_cache, block_table=torch.from_numpy(bt),
                      seq_lens=torch.tensor(ctx, dtype=torch.int32),
                      query_start_loc=torch.from_numpy(qsl), softmax_scale=float(np.float32(softmax_scale)),
                      causal=causal, window=window, window_expand_to_chunk=window_expand_to_chunk,
                      landmark_chunk=landmark_chunk, block_mask=block_mask, block_mask_tile=block_mask_tile,
                      scales=scales, out_heads_major=out_heads_major, dense_k=dense_k, dense_v=dense_v,
                      info=info, max_q_len=max(q_len) if q_len else 0,
                      min_q_len=min((x for x in q_len if x > 0), default=0))


# ---------------------------------------------------------------------------
# The five workloads (the page-derived shapes: Llama-3.1-8B attention heads,
# Hq 32 / Hkv 8 / d 128, 64-token pages, MTP q_len 1-4, 512-token prefill
# chunks, 128x128 block-sparse FP8 prefill, 4096-key sliding window with
# 64-token landmark chunks).
# ---------------------------------------------------------------------------

def tiny_hybrid(seed: int = 1, poison: bool = True, kv_layout: str = "NHD") -> PagedBatch:
    """fp32, Hq 4 / Hkv 1 / d 64, 16-token pages in a 64-page pool: two decode
    sequences (ctx 37 and 100) and a 16-token chunk over 48 history tokens."""
    rng = np.random.default_rng(seed)
    return build_batch(rng, name="tiny_hybrid_f32", kind="f32", Hq=4, Hkv=1, d=64, page_size=16,
                       ctx=[37, 100, 64], q_len=[1, 1, 16], num_pages=64, poison=poison,
                       keep_dense=True, kv_layout=kv_layout)


def decode_ctx_lengths(rng, batch: int, lo: int, hi: int) -> np.ndarray:
    """Log-uniform context lengths in [lo, hi], rounded."""
    u = rng.uniform(math.log(lo), math.log(hi), size=batch)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)


def splitk_decode(q_len=1, kv_layout: str = "NHD", seed: int = 2, batch: int = 64,
                  ctx_lo: int = 128, ctx_hi: int = 32768, poison: bool = True,
                  q_gain: float = 1.0, keep_dense: bool = False, kind: str = "bf16",
                  quant_mode: str = "tensor", q_quant: str = "token_head") -> PagedBatch:
    """Llama-3.1-8B attention shape, log-uniform contexts 128..32768,
    64-token pages, q_len in {1, 2, 4} (an int) or a per-sequence list (mixed MTP).
    bf16, or e4m3 (K/V scales per `quant_mode`, Q scales per `q_quant`: the
    decode variant scales Q per (token, head) and K/V per tensor)."""
    rng = np.random.default_rng(seed)
    ctx = decode_ctx_lengths(rng, batch, ctx_lo, ctx_hi)
    if isinstance(q_len, (list, tuple, np.ndarray)):
        ql = [int(x) for x in q_len]
        q_seed = 299
    else:
        ql = [int(q_len)] * batch
        q_seed = 200 + int(q_len)
    tag = "" if kind == "bf16" else f"_{kind}_{q_quant}_{quant_mode}"
    return build_batch(rng, name=f"splitk_decode_q{q_len if isinstance(q_len, int) else 'mix'}_{kv_layout}{tag}",
                       kind=kind, Hq=32, Hkv=8, d=128, page_size=64, ctx=ctx, q_len=ql,
                       kv_layout=kv_layout, q_rng=np.random.default_rng(q_seed), q_gain=q_gain,
                       poison=poison, keep_dense=keep_dense,
                       quant_mode=quant_mode if kind == "e4m3" else None,
                       q_quant=q_quant if kind == "e4m3" else "tensor")


def replay_variants(n: int = 4, batch: int = 16, total_q: int = 32, max_q_len: int = 4, ctx_lo: int = 64,
                    ctx_hi: int = 6000, seed: int = 9, kind: str = "bf16"):
    """Batches that share one set of buffers (Q, K/V caches, block table,
    seq_lens, query_start_loc of fixed shapes) but differ in their contents:
    each variant draws new context lengths, new q_len (summing to the same
    total_q, zeros allowed) and a new page permutation over the same cache,
    as a serving loop replaying one captured graph would.  Returns the list
    of PagedBatch (variant 0 owns the buffers' initial contents)."""
    rng = np.random.default_rng(seed)
    page_size, Hq, Hkv, d = 64, 32, 8, 128
    max_pages = -(-ctx_hi // page_size)
    num_pages = batch * max_pages
    base = None
    out = []
    for v in range(n):
        # q_len: total_q spread over the sequences, each at most max_q_len
        ql = np.zeros(batch, dtype=np.int64)
        for _ in range(total_q):
            free = np.nonzero(ql < max_q_len)[0]
            ql[rng.choice(free)] += 1
        ctx = np.maximum(decode_ctx_lengths(rng, batch, ctx_lo, ctx_hi), ql)
        if base is None:
            base = build_batch(rng, name="replay_v0", kind=kind, Hq=Hq, Hkv=Hkv, d=d, page_size=page_size,
                               ctx=[max_pages * page_size] * batch, q_len=[total_q // batch] * batch,
                               num_pages=num_pages, poison=False, quant_mode="tensor" if kind == "e4m3" else None)
        perm = rng.permutation(num_pages)
        bt = np.full((batch, max_pages), -1, dtype=np.int32)
        off = 0
        for b in range(batch):
            npg = -(-int(ctx[b]) // page_size)
            bt[b, :npg] = perm[off:off + npg]
            off += npg
        qsl = np.zeros(batch + 1, dtype=np.int32)
        qsl[1:] = np.cumsum(ql)
        kw = dict(base.__dict__)
        kw.update(name=f"replay_v{v}", block_table=torch.from_numpy(bt),
                  seq_lens=torch.from_numpy(ctx.astype(np.int32)), query_start_loc=torch.from_numpy(qsl),
                  max_q_len=max_q_len, min_q_len=0)
        out.append(PagedBatch(**kw))
    return out


def uniform_decode(ctx: int = 4096, batch: int = 64, q_len: int = 1, seed: int = 6, poison: bool = True,
                   kind: str = "bf16") -> PagedBatch:
    """Decode batch whose sequences all hold `ctx` keys (Llama-3.1-8B heads,
    64-token pages in a random permutation): the shape a static split suits."""
    rng = np.random.default_rng(seed)
    return build_batch(rng, name=f"uniform_decode_{ctx}_q{q_len}", kind=kind, Hq=32, Hkv=8, d=128,
                       page_size=64, ctx=[ctx] * batch, q_len=[q_len] * batch, poison=poison,
                       quant_mode="tensor" if kind == "e4m3" else None,
                       q_quant="token_head" if kind == "e4m3" else "tensor")


def hybrid_chunked(seed: int = 3, chunk_last: bool = False, poison: bool = True,
                   batch: int = 64, chunk: int = 512, history: int = 8192,
                   dec_lo: int = 1024, dec_hi: int = 16384, kv_layout: str = "NHD") -> PagedBatch:
    """bf16, one 512-token chunk over 8192 history tokens plus 63 decode
    sequences with contexts uniform in 1024..16384, packed varlen."""
    rng = np.random.default_rng(seed)
    dec = rng.integers(dec_lo, dec_hi + 1, size=batch - 1)
    ctx = [history + chunk] + [int(c) for c in dec]
    ql = [chunk] + [1] * (batch - 1)
    if chunk_last:
        ctx = ctx[1:] + ctx[:1]
        ql = ql[1:] + ql[:1]
    return build_batch(rng, name="hybrid_chunked" + ("_chunk_last" if chunk_last else ""), kind="bf16",
                       Hq=32, Hkv=8, d=128, page_size=64, ctx=ctx, q_len=ql, kv_layout=kv_layout,
                       poison=poison)


def sparse_prefill(kind: str = "e4m3", quant_mode: Optional[str] = "tensor", kv_layout: str = "NHD",
                   mask: bool = True, seed: int = 4, batch: int = 2, seq_len: int = 8192,
                   poison: bool = True, skip_target: float = 0.74) -> PagedBatch:
    """Causal prefill, batch 2 x 8192 tokens, Hq 32 / Hkv 8 / d 128, 64-token
    pages; e4m3 with per-tensor or per-(page, head) scales, or bf16.  With
    `mask`, a 128x128 tile block mask keeps the diagonal and skips each
    off-diagonal causal tile with probability chosen so that about
    `skip_target` of all causal tiles are skipped."""
    rng = np.random.default_rng(seed)
    ctx = [seq_len] * batch
    nqt = -(-seq_len // 128)
    n_causal = nqt * (nqt + 1) // 2
    p_skip = min(1.0, skip_target * n_causal / (n_causal - nqt)) if mask else None
    return build_batch(rng, name=f"sparse_prefill_{kind}_{quant_mode}_{kv_layout}_{'mask' if mask else 'dense'}",
                       kind=kind, Hq=32, Hkv=8, d=128, page_size=64, ctx=ctx, q_len=ctx,
                       kv_layout=kv_layout, quant_mode=quant_mode if kind == "e4m3" else None,
                       poison=poison, block_mask_skip=p_skip)


def sliding_window(decode: bool = False, window: int = 4096, landmark_chunk: int = 64,
                   seed: int = 5, seq_len: Optional[int] = None, poison: bool = True) -> PagedBatch:
    """bf16, B 1, Hq 32 / Hkv 8 / d 128, Lq = Lk = 8192, window 4096 with
    expand_to_chunk, landmark every 64 keys, contiguous K/V passed as NHD pages
    of 64 with an identity block table, outputs (B, Hq, Lq, d) and (B, Hq, Lq).
    decode=True: one query over a 131072-key context (window 0 and landmark 0
    give the plain full-context decode)."""
    rng = np.random.default_rng(seed)
    if decode:
        L = seq_len or 131072
        ctx, ql = [L], [1]
    else:
        L = seq_len or 8192
        ctx, ql = [L], [L]
    return build_batch(rng, name=f"sliding_window_{'decode' if decode else 'fwd'}_w{window}",
                       kind="bf16", Hq=32, Hkv=8, d=128, page_size=64, ctx=ctx, q_len=ql,
                       identity_pages=True, poison=poison, window=window,
                       window_expand_to_chunk=True, landmark_chunk=landmark_chunk,
                       out_heads_major=True)
