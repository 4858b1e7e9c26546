"""The allocation-free entry point against paged_attn_fwd, through the C ABI.

paged_attn_fwd_noalloc runs the same kernels on the library's own scratch
array instead of a caller workspace, so its outputs must equal those of
paged_attn_fwd bit for bit (same task map, same arithmetic), and both must
meet the oracle's tolerances.  Two calls in a row share the device's scratch
array: the second, smaller batch must not see anything the first left there.
"""
import numpy as np
import pytest
import torch

from attention_paged_kv_attn_amd import binding as B
from attention_paged_kv_attn_amd import workloads as W
from oracle import taskmap
from tests.oracle_helpers import run_oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-3), "e4m3": (4e-2, 1e-3), "f32": (1e-5, 1e-5)}
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def _outputs(g):
    dt = torch.float32 if g.kind == "f32" else torch.bfloat16
    return (torch.full((g.total_q, g.num_q_heads, g.head_dim), float("nan"), dtype=dt, device=DEV),
            torch.full((g.total_q, g.num_q_heads), float("nan"), dtype=torch.float32, device=DEV))


def _both(batch, **kw):
    """(out, lse) of paged_attn_fwd and of paged_attn_fwd_noalloc on one batch."""
    g = batch.to(DEV)
    o1, l1 = _outputs(g)
    o2, l2 = _outputs(g)
    say(f"  {batch.name}: total_q={g.total_q} B={g.num_seqs} kw={kw}")
    B.run_batch(g, out=o1, lse=l1, **kw)
    B.run_batch(g, out=o2, lse=l2, noalloc=True, **kw)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def _slots(b, force):
    """Partial slots a forced split of `force` units per worker needs."""
    P = B.paged_attn_device_info(0)["default_workers"]
    tm = taskmap.build(b.seq_lens.numpy(), b.query_start_loc.numpy(), Hq=b.num_q_heads, Hkv=b.num_kv_heads,
                       num_workers=P, force_split_units=force, causal=b.causal)
    return max(1, tm["n_slots"])


def _check(batch, o1, l1, o2, l2, rows=None):
    a1, a2 = o1.float().cpu().numpy(), o2.float().cpu().numpy()
    b1, b2 = l1.cpu().numpy(), l2.cpu().numpy()
    assert not np.isnan(a1).any() and not np.isnan(a2).any(), "rows left unwritten"
    assert np.array_equal(a1, a2, equal_nan=False), "O differs from paged_attn_fwd"
    assert np.array_equal(b1, b2), "LSE differs from paged_attn_fwd"
    O, L = run_oracle(batch, rows=rows)
    sel = np.ones(batch.total_q, bool) if rows is None else rows
    to, tl = TOL[batch.kind]
    eo = float(np.abs(a2[sel] - O[sel]).max())
    fin = np.isfinite(L[sel])
    assert np.array_equal(np.isneginf(b2[sel]), ~fin)
    el = float(np.abs(b2[sel][fin] - L[sel][fin]).max()) if fin.any() else 0.0
    say(f"  {batch.name}: bit-identical to paged_attn_fwd; oracle max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= to and el <= tl


def test_noalloc_matches_fwd_on_two_calls_second_smaller():
    # first call: the split-K decode batch (64 sequences, ctx up to 32768),
    # small-Q-block build with 16-row partial slots
    big = W.splitk_decode(q_len=1, seed=2)
    _check(big, *_both(big, max_q_len=1))
    # second call, smaller and of another shape: a hybrid chunk + decodes on the
    # general build (128-row partial slots), forced to split so partials and
    # Combine read the scratch array
    small = W.hybrid_chunked(batch=12, chunk=200, history=700, dec_lo=100, dec_hi=2000)
    _check(small, *_both(small, force_split_units=2, max_partial_slots=_slots(small, 2)))
    # and the natural split of the same batch
    _check(small, *_both(small))


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    b = W.splitk_decode(q_len=1, batch=4, ctx_lo=64, ctx_hi=300).to(DEV)
    o, l = _outputs(b)
    # 8192 workers: 16384 partial slots of 128 rows is far beyond the scratch array
    with pytest.raises(B.PagedAttnError) as e:
        B.run_batch(b, out=o, lse=l, noalloc=True, num_workers=8192)
    assert e.value.status == B.PA_ERR_SCRATCH
    need = B.paged_attn_workspace_size(B.make_params(
        num_seqs=b.num_seqs, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=b.page_size,
        num_pages=b.num_pages, max_pages_per_seq=b.block_table.shape[1], total_q=b.total_q,
        softmax_scale=b.softmax_scale, num_workers=8192))
    assert need > B.NOALLOC_SCRATCH_BYTES
    torch.cuda.synchronize()
    assert torch.isnan(o).all()                  # nothing was launched
