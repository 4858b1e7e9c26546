"""ctypes binding of libpaged_attn.so — argument marshalling only.

Every entry point of include/paged_attn.h is exposed under the same name.
torch supplies device memory (inputs, outputs, workspace) and the stream; all
computation runs in the library's HIP kernels.  If the library is missing the
functions raise; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaged_attn.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(5)
PA_F32, PA_BF16, PA_F8E4M3, PA_U8 = range(4)
PA_SCALE_NONE, PA_SCALE_PER_TENSOR, PA_SCALE_PER_PAGE_HEAD = range(3)
PA_SCALE_Q_PER_TOKEN_HEAD = 4
PA_SPLIT_DYNAMIC, PA_SPLIT_STATIC = range(2)
PA_PAIR_WEIGHT_SMALL, PA_PAIR_WEIGHT_GENERAL = 60, 50

EXPORTS = ("paged_attn_fwd", "paged_attn_workspace_size", "paged_attn_workspace_layout",
           "paged_attn_validate_host", "paged_attn_device_info", "paged_attn_status_string",
           "paged_attn_last_hip_error", "paged_attn_kernel_timing", "paged_attn_kernel_timing_read",
           "paged_attn_plan_split", "paged_attn_fwd_noalloc")
NOALLOC_SCRATCH_BYTES = 72 << 20
PA_ERR_SCRATCH = 5


class pa_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class pa_scales(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("q_scale", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class pa_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages",
        "max_pages_per_seq", "block_table_stride", "total_q")] + [("softmax_scale", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in (
            "causal", "window", "window_expand_to_chunk", "landmark_chunk", "block_mask_tile",
            "num_workers", "split_min_units", "force_split_units", "max_partial_slots", "flags",
            "split_mode", "static_splits", "max_q_len", "min_q_len", "pair_weight", "fused_combine",
            "qblock_per_kv_head")]


class pa_workspace_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "header", "seq_qb_base", "qb_desc", "unit_prefix", "n_splits", "slot_base", "combine_list",
        "done", "partial_lse", "partial_o", "total")] + [
        ("n_qb_max", ctypes.c_int32), ("max_slots", ctypes.c_int32), ("num_workers", ctypes.c_int32),
        ("slot_rows", ctypes.c_int32), ("qblock_heads", ctypes.c_int32)]


class pa_device_info(ctypes.Structure):
    _fields_ = [("compute_units", ctypes.c_int32), ("lds_bytes_per_workgroup", ctypes.c_int32),
                ("default_workers", ctypes.c_int32), ("arch", ctypes.c_char * 64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpaged_attn.so (built in-tree by attention_paged_kv_attn_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m attention_paged_kv_attn_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.paged_attn_fwd.argtypes = [P(pa_tensor), P(pa_tensor), P(pa_tensor), ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, P(pa_tensor), P(pa_scales),
                                     P(pa_tensor), P(pa_tensor), P(pa_params), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
        L.paged_attn_fwd_noalloc.argtypes = [P(pa_tensor), P(pa_tensor), P(pa_tensor), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, P(pa_tensor), P(pa_scales),
                                             P(pa_tensor), P(pa_tensor), P(pa_params), ctypes.c_void_p]
        L.paged_attn_workspace_size.argtypes = [P(pa_params), P(ctypes.c_size_t)]
        L.paged_attn_workspace_layout.argtypes = [P(pa_params), P(pa_workspace_layout)]
        L.paged_attn_validate_host.argtypes = [P(pa_params), ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32]
        L.paged_attn_device_info.argtypes = [ctypes.c_int32, P(pa_device_info)]
        L.paged_attn_plan_split.argtypes = [P(pa_params), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                            P(ctypes.c_int32), P(ctypes.c_int32)]
        L.paged_attn_status_string.argtypes = [ctypes.c_int32]
        L.paged_attn_status_string.restype = ctypes.c_char_p
        L.paged_attn_last_hip_error.restype = ctypes.c_int32
        L.paged_attn_kernel_timing.argtypes = [ctypes.c_int32]
        L.paged_attn_kernel_timing_read.argtypes = [P(ctypes.c_float)] * 3 + [P(ctypes.c_int32)]
        for name in EXPORTS:
            if name != "paged_attn_status_string" and name != "paged_attn_last_hip_error":
                getattr(L, name).restype = ctypes.c_int32
        _lib = L
    return _lib


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().paged_attn_status_string(status).decode()
        extra = ""
        if status == PA_ERR_HIP:
            extra = f" (hip error {lib().paged_attn_last_hip_error()})"
        super().__init__(f"{where}: {msg}{extra}")
        self.status = status


def _check(status: int, where: str):
    if status != PA_OK:
        raise PagedAttnError(status, where)


_DT = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.float8_e4m3fn: PA_F8E4M3, torch.uint8: PA_U8}


def as_pa_tensor(t: torch.Tensor, shape=None, strides=None) -> pa_tensor:
    """Describe a torch tensor (or a logical re-view of it via shape/strides)."""
    shape = list(t.shape) if shape is None else list(shape)
    strides = list(t.stride()) if strides is None else list(strides)
    pt = pa_tensor()
    pt.data = t.data_ptr()
    pt.dtype = _DT[t.dtype]
    pt.rank = len(shape)
    for i, (s, st) in enumerate(zip(shape, strides)):
        pt.shape[i] = int(s)
        pt.stride[i] = int(st)
    return pt


def kv_logical(cache: torch.Tensor, kv_layout: str) -> pa_tensor:
    """NHD [pages, slot, head, d] as is; HND [pages, head, slot, d] with strides permuted."""
    if kv_layout == "NHD":
        return as_pa_tensor(cache)
    if kv_layout == "HND":
        P_, H, S, D = cache.shape
        s = cache.stride()
        return as_pa_tensor(cache, (P_, S, H, D), (s[0], s[2], s[1], s[3]))
    raise ValueError(kv_layout)


def make_params(*, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                max_pages_per_seq, total_q, softmax_scale, block_table_stride=None, causal=True,
                window=0, window_expand_to_chunk=True, landmark_chunk=0, block_mask_tile=128,
                num_workers=0, split_min_units=0, force_split_units=0, max_partial_slots=0,
                split_mode=PA_SPLIT_DYNAMIC, static_splits=0, max_q_len=0, min_q_len=0, pair_weight=0,
                fused_combine=0, qblock_per_kv_head=0) -> pa_params:
    p = pa_params()
    p.num_seqs, p.num_q_heads, p.num_kv_heads, p.head_dim = num_seqs, num_q_heads, num_kv_heads, head_dim
    p.page_size, p.num_pages, p.max_pages_per_seq = page_size, num_pages, max_pages_per_seq
    p.block_table_stride = max_pages_per_seq if block_table_stride is None else block_table_stride
    p.total_q = total_q
    p.softmax_scale = softmax_scale
    p.causal, p.window, p.window_expand_to_chunk = int(causal), window, int(window_expand_to_chunk)
    p.landmark_chunk, p.block_mask_tile = landmark_chunk, block_mask_tile
    p.num_workers, p.split_min_units, p.force_split_units = num_workers, split_min_units, force_split_units
    p.max_partial_slots, p.flags = max_partial_slots, 0
    p.split_mode, p.static_splits = split_mode, static_splits
    p.max_q_len = max_q_len
    p.min_q_len = min_q_len
    p.pair_weight = pair_weight
    p.fused_combine = int(fused_combine)
    p.qblock_per_kv_head = int(qblock_per_kv_head)
    return p


def paged_attn_workspace_size(params: pa_params) -> int:
    n = ctypes.c_size_t()
    _check(lib().paged_attn_workspace_size(ctypes.byref(params), ctypes.byref(n)), "paged_attn_workspace_size")
    return n.value


def paged_attn_workspace_layout(params: pa_params) -> pa_workspace_layout:
    lay = pa_workspace_layout()
    _check(lib().paged_attn_workspace_layout(ctypes.byref(params), ctypes.byref(lay)), "paged_attn_workspace_layout")
    return lay


def paged_attn_validate_host(params: pa_params, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                             block_table: torch.Tensor, block_mask: Optional[torch.Tensor] = None) -> int:
    """Returns the pa_status (host tensors, int32 contiguous; block_mask dense u8)."""
    for t in (seq_lens, query_start_loc, block_table):
        assert t.device.type == "cpu" and t.dtype == torch.int32 and t.is_contiguous()
    mh = mq = mk = 0
    mptr = None
    if block_mask is not None:
        assert block_mask.device.type == "cpu" and block_mask.is_contiguous()
        _, mh, mq, mk = block_mask.shape
        mptr = block_mask.data_ptr()
    return lib().paged_attn_validate_host(ctypes.byref(params), seq_lens.data_ptr(),
                                          query_start_loc.data_ptr(), block_table.data_ptr(), mptr,
                                          mh, mq, mk)


def paged_attn_plan_split(params: pa_params, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                          has_block_mask: bool = False):
    """(split_mode, static_splits) the library's split policy picks for host metadata."""
    sl = seq_lens.detach().to("cpu", torch.int32).contiguous()
    qs = query_start_loc.detach().to("cpu", torch.int32).contiguous()
    mode, S = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().paged_attn_plan_split(ctypes.byref(params), sl.data_ptr(), qs.data_ptr(), int(has_block_mask),
                                       ctypes.byref(mode), ctypes.byref(S)), "paged_attn_plan_split")
    return mode.value, S.value


def paged_attn_device_info(device: int = 0) -> dict:
    info = pa_device_info()
    _check(lib().paged_attn_device_info(device, ctypes.byref(info)), "paged_attn_device_info")
    return {"compute_units": info.compute_units, "lds_bytes_per_workgroup": info.lds_bytes_per_workgroup,
            "default_workers": info.default_workers, "arch": info.arch.decode()}


def paged_attn_status_string(status: int) -> str:
    return lib().paged_attn_status_string(status).decode()


def paged_attn_last_hip_error() -> int:
    return lib().paged_attn_last_hip_error()


def paged_attn_kernel_timing(enable: bool) -> None:
    _check(lib().paged_attn_kernel_timing(int(enable)), "paged_attn_kernel_timing")


def paged_attn_kernel_timing_read():
    """(ms_assign, ms_attention, ms_combine, calls) summed since the last read."""
    a, b, c = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    n = ctypes.c_int32()
    _check(lib().paged_attn_kernel_timing_read(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                               ctypes.byref(n)), "paged_attn_kernel_timing_read")
    return a.value, b.value, c.value, n.value


def paged_attn_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_table: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                   block_mask: Optional[torch.Tensor] = None, scales: Optional[dict] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, *,
                   softmax_scale: Optional[float] = None, kv_layout: str = "NHD", causal: bool = True,
                   window: int = 0, window_expand_to_chunk: bool = True, landmark_chunk: int = 0,
                   block_mask_tile: int = 128, num_workers: int = 0, split_min_units: int = 0,
                   force_split_units: int = 0, max_partial_slots: int = 0, split: str = "dynamic",
                   static_splits: int = 0, max_q_len: int = 0, min_q_len: int = 0, pair_weight: int = 0,
                   fused_combine: bool = False, workspace: Optional[torch.Tensor] = None, stream=None,
                   noalloc: bool = False, qblock_per_kv_head: bool = False):
    """Run the library on torch tensors; returns (out, lse, workspace).

    noalloc: call paged_attn_fwd_noalloc (the library's own scratch array is
    the workspace; `workspace` must be None and None is returned for it).

    q [total_q, Hq, d]; k_cache/v_cache NHD [pages, page_size, Hkv, d] or HND
    [pages, Hkv, page_size, d]; block_table int32 [B, max_pages]; seq_lens int32
    [B]; query_start_loc int32 [B + 1]; block_mask u8 [B, H_m, n_q_tiles,
    n_k_tiles]; scales {"mode": "tensor"|"page_head", "q","k","v": fp32 device
    tensors}.  out [total_q, Hq, d] (f32 for f32 inputs, else bf16) and lse f32
    [total_q, Hq] may be strided views; missing buffers are allocated here with
    torch (the library itself allocates nothing).  split: "dynamic" (Assign's
    task map), "static" (static_splits per Q-block) or "auto" (the library's
    policy on host copies of seq_lens / query_start_loc).
    """
    total_q, Hq, d = q.shape
    if kv_layout == "NHD":
        num_pages, page_size, Hkv, _ = k_cache.shape
    else:
        num_pages, Hkv, page_size, _ = k_cache.shape
    B = seq_lens.shape[0]
    assert block_table.dtype == torch.int32 and block_table.stride(1) == 1
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    params = make_params(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, page_size=page_size,
                         num_pages=num_pages, max_pages_per_seq=block_table.shape[1],
                         block_table_stride=block_table.stride(0), total_q=total_q,
                         softmax_scale=softmax_scale, causal=causal, window=window,
                         window_expand_to_chunk=window_expand_to_chunk, landmark_chunk=landmark_chunk,
                         block_mask_tile=block_mask_tile, num_workers=num_workers,
                         split_min_units=split_min_units, force_split_units=force_split_units,
                         max_partial_slots=max_partial_slots, max_q_len=max_q_len, min_q_len=min_q_len,
                         pair_weight=pair_weight,
                         fused_combine=fused_combine, qblock_per_kv_head=qblock_per_kv_head)
    if split == "auto":
        params.split_mode, params.static_splits = paged_attn_plan_split(params, seq_lens, query_start_loc,
                                                                        block_mask is not None)
    elif split == "static":
        params.split_mode, params.static_splits = PA_SPLIT_STATIC, static_splits
    elif split != "dynamic":
        raise ValueError("split must be 'dynamic', 'static' or 'auto'")
    out_dtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((total_q, Hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    if noalloc:
        if workspace is not None:
            raise ValueError("the no-allocation entry point takes no workspace")
    else:
        need = paged_attn_workspace_size(params)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    sc = None
    if scales is not None:
        sc = pa_scales()
        sc.mode = {"tensor": PA_SCALE_PER_TENSOR, "page_head": PA_SCALE_PER_PAGE_HEAD}[scales["mode"]]
        if scales.get("q_mode", "tensor") == "token_head":
            qs = scales["q"]
            if qs.dtype != torch.float32 or not qs.is_contiguous() or qs.numel() != total_q * Hq:
                raise ValueError("per-(token, head) Q scales must be contiguous fp32 [total_q, Hq]")
            sc.mode |= PA_SCALE_Q_PER_TOKEN_HEAD
        elif scales.get("q_mode", "tensor") != "tensor":
            raise ValueError("q_mode must be 'tensor' or 'token_head'")
        sc.q_scale, sc.k_scale, sc.v_scale = (scales["q"].data_ptr(), scales["k"].data_ptr(),
                                              scales["v"].data_ptr())
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    qt, kt, vt = as_pa_tensor(q), kv_logical(k_cache, kv_layout), kv_logical(v_cache, kv_layout)
    ot, lt = as_pa_tensor(out), as_pa_tensor(lse)
    mt = as_pa_tensor(block_mask) if block_mask is not None else None
    common = (ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), block_table.data_ptr(),
              seq_lens.data_ptr(), query_start_loc.data_ptr(), ctypes.byref(mt) if mt is not None else None,
              ctypes.byref(sc) if sc is not None else None, ctypes.byref(ot), ctypes.byref(lt),
              ctypes.byref(params))
    if noalloc:
        _check(lib().paged_attn_fwd_noalloc(*common, ctypes.c_void_p(stream)), "paged_attn_fwd_noalloc")
        return out, lse, None
    st = lib().paged_attn_fwd(*common, workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(stream))
    _check(st, "paged_attn_fwd")
    return out, lse, workspace


def run_batch(batch, *, out=None, lse=None, workspace=None, **kw):
    """paged_attn_fwd on a workloads.PagedBatch that already lives on the GPU."""
    if out is None and batch.out_heads_major:
        B = batch.num_seqs
        assert B == 1, "heads-major output layout is built for a single sequence"
        full_o = torch.empty((1, batch.num_q_heads, batch.total_q, batch.head_dim),
                             dtype=torch.float32 if batch.kind == "f32" else torch.bfloat16, device=batch.q.device)
        full_l = torch.empty((1, batch.num_q_heads, batch.total_q), dtype=torch.float32, device=batch.q.device)
        out = full_o[0].permute(1, 0, 2)
        lse = full_l[0].permute(1, 0)
    args = dict(softmax_scale=batch.softmax_scale, kv_layout=batch.kv_layout, causal=batch.causal,
                max_q_len=batch.max_q_len, min_q_len=batch.min_q_len,
                window=batch.window, window_expand_to_chunk=batch.window_expand_to_chunk,
                landmark_chunk=batch.landmark_chunk, block_mask_tile=batch.block_mask_tile)
    args.update(kw)
    return paged_attn_fwd(batch.q, batch.k_cache, batch.v_cache, batch.block_table, batch.seq_lens,
                          batch.query_start_loc, batch.block_mask, batch.scales, out, lse,
                          workspace=workspace, **args)
