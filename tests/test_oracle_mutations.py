"""The pins must catch plausible mistakes: each test plants one mistake in a
copy of an oracle function (on the CPU, never in the HIP path) and checks that
the pin written for that part of the oracle fails on the copy and passes on
the real function."""
import inspect
import types

import numpy as np
import pytest

from attention_paged_kv_attn_amd import workloads as W
from oracle import attention as oracle_attention
from oracle import taskmap
from tests import test_oracle_attention as T_att
from tests import test_oracle_taskmap as T_map


def _mutant(module, func_name, old, new):
    """A copy of module.func_name whose source has `old` replaced by `new`."""
    src = inspect.getsource(getattr(module, func_name))
    assert src.count(old) == 1, (func_name, old)
    ns = dict(vars(module))
    exec(compile(src.replace(old, new), f"<mutant {func_name}>", "exec"), ns)
    return ns[func_name]


def test_taskmap_pin_catches_floor_for_ceil():
    ctx = W.decode_ctx_lengths(np.random.default_rng(5), 50, 64, 5000)
    qsl = np.arange(51)
    P = 64
    real = taskmap.build(ctx, qsl, Hq=32, Hkv=8, num_workers=P)
    assert real["U"] % P != 0                      # a load where floor and ceil differ
    T_map._check_invariants(real)
    broken = _mutant(taskmap, "build", "-(-U // P)", "U // P")
    tm = broken(ctx, qsl, Hq=32, Hkv=8, num_workers=P)
    with pytest.raises(AssertionError):
        T_map._check_invariants(tm)


def test_empty_row_pin_catches_nan_rows(monkeypatch):
    broken = _mutant(oracle_attention, "_softmax_rows", "o[empty] = 0.0", "o[empty] = np.nan")
    T_att.test_rows_without_visible_keys_inside_a_nonempty_span()      # the real oracle passes
    monkeypatch.setattr(oracle_attention, "_softmax_rows", broken)
    with pytest.raises(AssertionError):
        T_att.test_rows_without_visible_keys_inside_a_nonempty_span()


def test_empty_row_pin_catches_a_finite_lse(monkeypatch):
    broken = _mutant(oracle_attention, "_softmax_rows", "lse[empty] = -np.inf", "lse[empty] = 0.0")
    monkeypatch.setattr(oracle_attention, "_softmax_rows", broken)
    with pytest.raises(AssertionError):
        T_att.test_rows_without_visible_keys_inside_a_nonempty_span()
