"""Pins for the K/V append oracle (a pure bit copy)."""

import numpy as np
import pytest
import torch

from oracle import kv_append_bits, gather_sequence
from workloads import BlockPool

BS = 16


def test_token_by_token_append_rebuilds_the_sequence():
    """Append every token of three sequences one step at a time, with the slot
    the pool hands out; the final cache read back position by position is the
    original contiguous data, and no other slot was touched."""
    rng = np.random.default_rng(0)
    H, D, NB = 2, 8, 12
    lens = [5, 16, 33]
    data = [rng.standard_normal((L, H, D)).astype(np.float32) for L in lens]
    pool = BlockPool(NB, rng.permutation(NB), BS)
    for b in range(3):
        pool.new_sequence(b)
    cache = np.full((NB, H, BS, D), np.nan, dtype=np.float32)
    written = np.zeros((NB, BS), dtype=bool)
    for step in range(max(lens)):
        rows, slots = [], []
        for b in range(3):
            if step < lens[b]:
                s = pool.append_token(b)
                rows.append(data[b][step]); slots.append(s)
                written[s // BS, s % BS] = True
            else:
                rows.append(np.zeros((H, D), np.float32)); slots.append(-1)
        cache = kv_append_bits(cache, np.stack(rows), np.array(slots))
    for b in range(3):
        tab = np.array(pool.tables[b])
        back = gather_sequence(cache, tab, lens[b], "f32")
        np.testing.assert_array_equal(back, data[b].astype(np.float64))
    assert np.isnan(cache.transpose(0, 2, 1, 3)[~written]).all()


def test_bits_are_copied_not_values():
    """NaN payloads and -0.0 survive: the append moves bit patterns."""
    cache = np.zeros((2, 1, BS, 4), dtype=np.uint16)
    new = np.array([[[0x7E01, 0x8000, 0xFFFF, 0x0001]]], dtype=np.uint16)
    out = kv_append_bits(cache, new, np.array([17]))
    assert np.array_equal(out[1, 0, 1], new[0, 0])
    out[1, 0, 1] = 0
    assert not out.any()


def test_minus_one_slots_are_skipped_and_input_unchanged():
    cache = np.arange(2 * 1 * BS * 2, dtype=np.float32).reshape(2, 1, BS, 2)
    keep = cache.copy()
    new = np.full((3, 1, 2), -5.0, np.float32)
    out = kv_append_bits(cache, new, np.array([-1, 3, -1]))
    assert np.array_equal(cache, keep)                       # not in place
    diff = np.argwhere(out != keep)
    assert {tuple(d[:3]) for d in diff} == {(0, 0, 3)}


def test_bad_slots_raise():
    cache = np.zeros((2, 1, BS, 2), np.float32)
    with pytest.raises(ValueError):
        kv_append_bits(cache, np.zeros((2, 1, 2), np.float32), np.array([4, 4]))
    with pytest.raises(IndexError):
        kv_append_bits(cache, np.zeros((1, 1, 2), np.float32), np.array([2 * BS]))


def test_matches_torch_index_copy():
    """A library scatter (torch.index_copy_ on the flattened slot axis) agrees."""
    rng = np.random.default_rng(1)
    NB, H, D, T = 7, 3, 8, 9
    cache = rng.standard_normal((NB, H, BS, D)).astype(np.float16)
    new = rng.standard_normal((T, H, D)).astype(np.float16)
    slots = rng.choice(NB * BS, size=T, replace=False)
    ours = kv_append_bits(cache, new, slots)
    t = torch.from_numpy(cache.copy()).permute(0, 2, 1, 3).reshape(NB * BS, H, D)
    t.index_copy_(0, torch.from_numpy(slots), torch.from_numpy(new))
    ref = t.reshape(NB, BS, H, D).permute(0, 2, 1, 3).numpy()
    assert np.array_equal(ours.view(np.uint16), ref.view(np.uint16))
