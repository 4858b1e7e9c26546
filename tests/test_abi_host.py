"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from attention_paged_kv_attn_amd import binding as B
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "paged_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(paged_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTS)


def test_status_strings():
    for s in range(6):
        assert B.paged_attn_status_string(s) != "unknown status"
    assert B.paged_attn_status_string(0) == "ok"


def _params(**kw):
    base = dict(num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, num_pages=6000,
                max_pages_per_seq=512, total_q=64, softmax_scale=0.0883883, num_workers=512)
    base.update(kw)
    return B.make_params(**base)


def test_workspace_size_closed_form():
    p = _params()
    lay = B.paged_attn_workspace_layout(p)
    n_qb_max = 8 * (64 + (64 * 4 + 127) // 128)
    assert lay.n_qb_max == n_qb_max and lay.max_slots == 1024 and lay.num_workers == 512
    assert lay.total == B.paged_attn_workspace_size(p)
    assert lay.partial_o >= lay.partial_lse + 1024 * 128 * 4
    assert lay.total >= lay.partial_o + 1024 * 128 * 128 * 4
    offs = [lay.header, lay.seq_qb_base, lay.qb_desc, lay.unit_prefix, lay.n_splits, lay.slot_base,
            lay.combine_list, lay.partial_lse, lay.partial_o, lay.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.slot_rows == 128                  # the general kernel build: 128-row Q-blocks
    # monotone in the sizes that drive it
    assert B.paged_attn_workspace_size(_params(total_q=4096)) > lay.total
    assert B.paged_attn_workspace_size(_params(num_workers=1024)) > lay.total


def test_partial_slots_follow_the_kernel_build():
    """A call whose Q-blocks are all known to be small (max_q_len * G <= 16, or
    a static split) gets 16-row partial slots; otherwise slots hold 128 rows."""
    # (Hq 32, Hkv 8: G = 4, two kv heads per wave.)  Sequence Q-blocks hold
    # max_q_len * Hq rows; they apply while max_q_len * G * Hkv / 4 <= 16
    for kw, rows, heads in ((dict(max_q_len=4), 16, 4), (dict(max_q_len=1), 32, 32), (dict(max_q_len=2), 64, 32),
                            (dict(max_q_len=1, qblock_per_kv_head=1), 16, 4), (dict(max_q_len=5), 128, 4),
                            (dict(min_q_len=32), 128, 4), (dict(split_mode=B.PA_SPLIT_STATIC, static_splits=2), 16, 4),
                            (dict(max_q_len=1, num_q_heads=12, num_kv_heads=6), 16, 2), ({}, 128, 4)):
        lay = B.paged_attn_workspace_layout(_params(**kw))
        assert (lay.slot_rows, lay.qblock_heads) == (rows, heads), kw
        assert lay.partial_o - lay.partial_lse >= lay.max_slots * rows * 4
        assert lay.total - lay.partial_o >= lay.max_slots * rows * 128 * 4
    small = B.paged_attn_workspace_size(_params(max_q_len=1, qblock_per_kv_head=1))
    assert small < B.paged_attn_workspace_size(_params()) // 4


def test_odd_worker_count_gets_slots_for_one_more_worker():
    assert B.paged_attn_workspace_layout(_params(num_workers=7)).max_slots == 16
    assert B.paged_attn_workspace_layout(_params(num_workers=8)).max_slots == 16
    assert B.paged_attn_workspace_layout(_params(num_workers=7, max_partial_slots=5)).max_slots == 5


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(num_kv_heads=5), dict(page_size=48),
                                 dict(num_q_heads=24, num_kv_heads=8), dict(block_mask_tile=100),
                                 dict(num_seqs=0), dict(max_pages_per_seq=0), dict(window=-1),
                                 dict(softmax_scale=0.0), dict(softmax_scale=-0.1),
                                 dict(softmax_scale=float("inf")), dict(softmax_scale=float("nan"))])
def test_bad_params_rejected(bad):
    p = _params(**bad)
    n = ctypes.c_size_t()
    st = B.lib().paged_attn_workspace_size(ctypes.byref(p), ctypes.byref(n))
    assert st in (B.PA_ERR_INVALID_ARG, B.PA_ERR_UNSUPPORTED)


def _fake(shape, dtype, addr=1 << 20):
    """A pa_tensor describing fake device memory (never dereferenced: every call
    below fails its checks before launching)."""
    t = B.pa_tensor()
    t.data = addr
    t.dtype = dtype
    t.rank = len(shape)
    st = 1
    strides = []
    for s in reversed(shape):
        strides.append(st)
        st *= s
    for i, (s, sd) in enumerate(zip(shape, reversed(strides))):
        t.shape[i] = s
        t.stride[i] = sd
    return t


def _call(q, k, v, out, lse, p, ws=1 << 24, ws_bytes=1 << 40, mask=None, scales=None, ptrs=(1 << 21,) * 3):
    by = ctypes.byref
    return B.lib().paged_attn_fwd(by(q) if q else None, by(k), by(v), ptrs[0], ptrs[1], ptrs[2],
                                  by(mask) if mask else None, by(scales) if scales else None,
                                  by(out), by(lse), by(p), ws, ws_bytes, None)


def _valid():
    p = _params(num_seqs=4, total_q=4, num_pages=100, max_pages_per_seq=16)
    q = _fake([4, 32, 128], B.PA_BF16)
    k = _fake([100, 64, 8, 128], B.PA_BF16)
    v = _fake([100, 64, 8, 128], B.PA_BF16)
    o = _fake([4, 32, 128], B.PA_BF16)
    l = _fake([4, 32], B.PA_F32)
    return q, k, v, o, l, p


def test_fwd_argument_errors_before_launch():
    q, k, v, o, l, p = _valid()
    assert _call(None, k, v, o, l, p) == B.PA_ERR_INVALID_ARG
    q2 = _fake([5, 32, 128], B.PA_BF16)
    assert _call(q2, k, v, o, l, p) == B.PA_ERR_INVALID_ARG                  # total_q mismatch
    o32 = _fake([4, 32, 128], B.PA_F32)
    assert _call(q, k, v, o32, l, p) == B.PA_ERR_UNSUPPORTED                 # bf16 in -> bf16 out
    k8 = _fake([100, 64, 8, 128], B.PA_F8E4M3)
    assert _call(q, k8, v, o, l, p) == B.PA_ERR_UNSUPPORTED                  # dtype mix
    kbad = _fake([100, 32, 8, 128], B.PA_BF16)
    assert _call(q, kbad, v, o, l, p) == B.PA_ERR_INVALID_ARG                # page_size mismatch
    assert _call(q, k, v, o, l, p, ws=0) == B.PA_ERR_WORKSPACE
    assert _call(q, k, v, o, l, p, ws=(1 << 24) + 16) == B.PA_ERR_WORKSPACE  # misaligned
    assert _call(q, k, v, o, l, p, ws_bytes=100) == B.PA_ERR_WORKSPACE
    assert _call(q, k, v, o, l, p, ptrs=(0, 1 << 21, 1 << 21)) == B.PA_ERR_INVALID_ARG
    qm = _fake([4, 32, 128], B.PA_BF16, addr=(1 << 20) + 2)
    assert _call(qm, k, v, o, l, p) == B.PA_ERR_INVALID_ARG                  # misaligned rows
    # fp8 needs scales, and per-(page, head) scales need pages of >= 64 keys
    q8, v8, = _fake([4, 32, 128], B.PA_F8E4M3), _fake([100, 64, 8, 128], B.PA_F8E4M3)
    assert _call(q8, k8, v8, o, l, p) == B.PA_ERR_INVALID_ARG
    sc = B.pa_scales()
    sc.mode = B.PA_SCALE_PER_PAGE_HEAD
    sc.q_scale = sc.k_scale = sc.v_scale = 1 << 22
    p16 = _params(num_seqs=4, total_q=4, num_pages=100, max_pages_per_seq=64, page_size=16)
    k16, v16 = _fake([100, 16, 8, 128], B.PA_F8E4M3), _fake([100, 16, 8, 128], B.PA_F8E4M3)
    assert _call(q8, k16, v16, o, l, p16, scales=sc) == B.PA_ERR_UNSUPPORTED
    # a block mask must be u8 with 1 or Hq heads
    m = _fake([4, 3, 2, 2], B.PA_U8)
    assert _call(q, k, v, o, l, p, mask=m) == B.PA_ERR_INVALID_ARG


def test_validate_host():
    ctx = torch.tensor([37, 100, 64], dtype=torch.int32)
    qsl = torch.tensor([0, 1, 2, 18], dtype=torch.int32)
    bt = torch.full((3, 7), -1, dtype=torch.int32)
    bt[0, :3] = torch.tensor([1, 2, 3])
    bt[1, :7] = torch.arange(4, 11)
    bt[2, :4] = torch.arange(11, 15)
    p = B.make_params(num_seqs=3, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, num_pages=64,
                      max_pages_per_seq=7, total_q=18, softmax_scale=0.125, num_workers=4)
    assert B.paged_attn_validate_host(p, ctx, qsl, bt) == B.PA_OK
    bad = bt.clone()
    bad[1, 6] = 64
    assert B.paged_attn_validate_host(p, ctx, qsl, bad) == B.PA_ERR_INVALID_ARG
    bad = bt.clone()
    bad[2, 3] = -1
    assert B.paged_attn_validate_host(p, ctx, qsl, bad) == B.PA_ERR_INVALID_ARG
    assert B.paged_attn_validate_host(p, ctx, torch.tensor([0, 1, 2, 17], dtype=torch.int32), bt) \
        == B.PA_ERR_INVALID_ARG
    short = torch.tensor([37, 100, 15], dtype=torch.int32)           # q_len 16 > seq_len 15
    assert B.paged_attn_validate_host(p, short, qsl, bt) == B.PA_ERR_INVALID_ARG
    mask = torch.ones((3, 1, 1, 1), dtype=torch.uint8)                # covers 128 keys only
    assert B.paged_attn_validate_host(p, ctx, qsl, bt, mask) == B.PA_OK
    long_ctx = torch.tensor([37, 100, 200], dtype=torch.int32)
    bt2 = torch.zeros((3, 13), dtype=torch.int32)
    p2 = B.make_params(num_seqs=3, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, num_pages=64,
                       max_pages_per_seq=13, total_q=18, softmax_scale=0.125, num_workers=4)
    assert B.paged_attn_validate_host(p2, long_ctx, qsl, bt2, mask) == B.PA_ERR_INVALID_ARG


def _plan(ctx, ql, *, Hq=32, Hkv=8, P=512, mask=False, **kw):
    import torch
    qsl = [0]
    for x in ql:
        qsl.append(qsl[-1] + x)
    params = B.make_params(num_seqs=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, page_size=64,
                           num_pages=1 << 20, max_pages_per_seq=max(1, -(-max(ctx) // 64)),
                           total_q=qsl[-1], softmax_scale=0.088, num_workers=P, **kw)
    return B.paged_attn_plan_split(params, torch.tensor(ctx, dtype=torch.int32),
                                   torch.tensor(qsl, dtype=torch.int32), mask)


def test_split_policy_choices():
    """The policy's documented rule on shapes worked out by hand:
    busiest worker under the dynamic map = max(8, ceil(U / P)) + 3 + 2 tiles,
    under a static cut = ceil(n_qb S / P) * ceil(T_max / S) (+ 2 when S > 1)."""
    rng = np.random.default_rng(2)
    loguni = np.clip(np.rint(np.exp(rng.uniform(np.log(128), np.log(32768), 64))), 128, 32768).astype(int)
    # ragged decode: a static cut leaves the longest sequence on one workgroup -> dynamic
    assert _plan(loguni.tolist(), [1] * 64) == (B.PA_SPLIT_DYNAMIC, 0)
    # uniform decode, 512 Q-blocks of 64 tiles on 512 workers: no split (64 <= 64 + 5)
    assert _plan([4096] * 64, [1] * 64) == (B.PA_SPLIT_STATIC, 1)
    # one 128K sequence, 8 Q-blocks of 2048 tiles: S = 64 gives 32 + 2 <= 32 + 5
    assert _plan([131072], [1], P=512) == (B.PA_SPLIT_STATIC, 64)
    # windowed 128K decode: the window starts on a 64-key boundary, so 64 tiles
    # per Q-block; at most ceil(64 / 8) = 8 splits of 8 tiles -> 8 + 2 = 10 <= max(8, 1) + 5
    assert _plan([131072], [1], window=4096, landmark_chunk=64) == (B.PA_SPLIT_STATIC, 8)
    # prefill rows (q_len * G > 16) and block masks are dynamic only
    assert _plan([4096] * 4, [512] * 4) == (B.PA_SPLIT_DYNAMIC, 0)
    assert _plan([4096] * 64, [1] * 64, mask=True) == (B.PA_SPLIT_DYNAMIC, 0)
    # MTP 4 with G = 4 is still one small Q-block per (b, g)
    assert _plan([4096] * 64, [4] * 64) == (B.PA_SPLIT_STATIC, 1)


def test_static_split_argument_checks():
    import torch
    params = B.make_params(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16, num_pages=8,
                           max_pages_per_seq=4, total_q=2, softmax_scale=0.125, num_workers=4,
                           split_mode=B.PA_SPLIT_STATIC, static_splits=0)
    n = ctypes.c_size_t()
    assert B.lib().paged_attn_workspace_size(ctypes.byref(params), ctypes.byref(n)) == B.PA_ERR_INVALID_ARG
    params.static_splits = 2
    assert B.lib().paged_attn_workspace_size(ctypes.byref(params), ctypes.byref(n)) == B.PA_OK
    params.split_mode = 7
    assert B.lib().paged_attn_workspace_size(ctypes.byref(params), ctypes.byref(n)) == B.PA_ERR_INVALID_ARG
