"""Per-step K/V append into a paged cache, on raw bits.

[P1] section 2.3: each decode step writes the new token's K and V at the
sequence's current length and then advances the length by one.  [P5]
section 4 (locate()): with paging the write goes to the flat slot
physical_block * block_size + offset.  A slot of -1 means "no token".

The append is a pure copy, so it is done on the stored bit patterns and the
result is compared bit for bit.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np


def kv_append_bits(cache, new, slot_mapping, block_size: int = 16) -> np.ndarray:
    """Return a copy of `cache` [NB, Hkv, bs, D] with `new` [T, Hkv, D] written.

    Both arrays are raw storage (any numpy dtype of the right width); for
    every token t with slot_mapping[t] >= 0 the K (or V) row of every head is
    placed at block slot // bs, offset slot % bs.  Slots must be distinct.
    """
    cache = np.array(cache, copy=True)
    new = np.asarray(new)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    nb, hkv, bs, d = cache.shape
    if bs != block_size or new.shape[1:] != (hkv, d) or new.shape[0] != slots.shape[0]:
        raise ValueError("shape mismatch")
    used = slots[slots >= 0]
    if len(np.unique(used)) != len(used):
        raise ValueError("duplicate slots")
    if len(used) and used.max() >= nb * bs:
        raise IndexError("slot outside the pool")
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        cache[slot // bs, :, slot % bs, :] = new[t]
    return cache
