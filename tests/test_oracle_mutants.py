"""Planted mistakes in the oracle (on the CPU): each must be caught by at
least one pin, showing that the pins constrain the oracle."""
import types

import numpy as np
import pytest

from oracle import pa_oracle as O
from tests.test_oracle_attention import ALL_PINS


def _mutant(**overrides):
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update(O.__dict__)
    m.__dict__.update(overrides)
    # the module-level functions resolve helpers through their globals, so
    # re-bind decode/decode_one to the mutant namespace
    for name in ("decode", "decode_one", "partition_partials", "combine_partials", "decode_partitioned"):
        f = O.__dict__[name]
        if name not in overrides:
            m.__dict__[name] = types.FunctionType(f.__code__, m.__dict__, name, f.__defaults__, f.__closure__)
    return m


def _off_by_one_offset(table, seq_len, block_size):
    pos = np.arange(int(seq_len))
    phys = np.asarray(table, dtype=np.int64)[pos // block_size]
    return phys, (pos + 1) % block_size


def _swapped_div_mod(table, seq_len, block_size):
    pos = np.arange(int(seq_len))
    tab = np.asarray(table, dtype=np.int64)
    return tab[(pos % block_size) % max(1, len([b for b in tab if b >= 0]))], pos // block_size


def _interleaved_heads(h, hq, hkv):
    return h % hkv


def _unnormalised(scores, values):
    m = scores.max()
    w = np.exp(scores - m)
    return w @ values


def _unscaled_one(q_row, k_pool, v_pool, table, seq_len, scale, kv_head, block_size):
    return O.decode_one(q_row, k_pool, v_pool, table, seq_len, 1.0, kv_head, block_size)


def _first_row_only(pool, phys, off, kv_head):
    return pool[phys, kv_head, np.zeros_like(off), :]


MUTANTS = {
    "offset_off_by_one": dict(positions_to_rows=_off_by_one_offset),
    "div_mod_swapped": dict(positions_to_rows=_swapped_div_mod),
    "gqa_interleaved": dict(kv_head_of=_interleaved_heads),
    "softmax_unnormalised": dict(_softmax_weighted_sum=_unnormalised),
    "scale_dropped": dict(decode_one=_unscaled_one),
    "gather_ignores_offset": dict(_gather=_first_row_only),
}


def _caught(mod):
    for pin in ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError):
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(**MUTANTS[name])
    assert _caught(mod) is not None, f"no pin catches mutant {name}"


def test_unmutated_passes_all_pins():
    assert _caught(_mutant()) is None
