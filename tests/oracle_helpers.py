"""Glue between the seeded workloads (torch tensors) and the oracle (NumPy)."""
import numpy as np
import torch


def stored_np(t: torch.Tensor, kind: str) -> np.ndarray:
    t = t.detach().cpu()
    if kind == "bf16":
        return t.view(torch.uint16).numpy()
    if kind == "e4m3":
        return t.view(torch.uint8).numpy()
    return t.numpy()


def oracle_scales(batch):
    if batch.scales is None:
        return None
    s = batch.scales
    k = s["k"].cpu().numpy()
    v = s["v"].cpu().numpy()
    if s["mode"] == "tensor":
        k, v = float(k[0]), float(v[0])
    q_mode = s.get("q_mode", "tensor")
    q = float(s["q"].cpu()[0]) if q_mode == "tensor" else s["q"].cpu().numpy()
    return {"mode": s["mode"], "q_mode": q_mode, "q": q, "k": k, "v": v}


def run_oracle(batch, **overrides):
    """oracle.attention.paged_attention on a workloads.PagedBatch."""
    from oracle.attention import paged_attention
    kw = dict(kind=batch.kind, softmax_scale=batch.softmax_scale, kv_layout=batch.kv_layout,
              causal=batch.causal, window=batch.window,
              window_expand_to_chunk=batch.window_expand_to_chunk,
              landmark_chunk=batch.landmark_chunk,
              block_mask=None if batch.block_mask is None else batch.block_mask.cpu().numpy(),
              block_mask_tile=batch.block_mask_tile, scales=oracle_scales(batch))
    kw.update(overrides)
    return paged_attention(stored_np(batch.q, batch.kind), stored_np(batch.k_cache, batch.kind),
                           stored_np(batch.v_cache, batch.kind), batch.block_table.cpu().numpy(),
                           batch.seq_lens.cpu().numpy(), batch.query_start_loc.cpu().numpy(), **kw)


def dequant64(t: torch.Tensor, scale=None) -> np.ndarray:
    """Widen stored values with torch (independent of the oracle's own upcast)."""
    x = t.detach().cpu().to(torch.float64).numpy()
    if scale is not None:
        x = x * scale
    return x
