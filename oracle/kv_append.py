"""Per-step K/V append into a paged cache, on raw bits.

[P1] section 2.3: each decode step writes the new token's K and V at the
sequence's current length and then advances the length by one.  [P5]
section 4 (locate()): with paging the write goes to the flat slot
physical_block * block_size + offset.  A slot of -1 means "no token".

The plain append is a pure copy, so it is done on the stored bit patterns
and the result is compared bit for bit.  The FP8 append quantises on write
([P5] section 7: 8-bit K/V with one scale per head; [P4]: FP8 KV needs
calibrated scales): its codes are decided in fp32, exactly as stated below,
so they too are compared bit for bit.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np

from .fp8_e4m3 import E4M3_MAX, encode_e4m3fn_rne


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


def kv_append_fp8(cache_codes, scales, new_values, slot_mapping, *, first_write: bool,
                  block_size: int = 16):
    """Quantise-on-write into an e4m3fn cache; returns new (codes, scales).

    cache_codes: uint8 [NB, Hkv, bs, D]; scales: float32 [NB, Hkv];
    new_values: float32 [T, Hkv, D] (the source values, widened exactly).
    For every token t with slot s = slot_mapping[t] in [0, NB * bs):
      * first_write and s % bs == 0 (the block's first token): the block's
        scale for head h becomes float32(max_d |x[t, h, d]|) / float32(448)
        in fp32 (1.0 when that max is 0); all such scales are set before any
        token is quantised;
      * every element becomes RNE(clamp(float32(x) / scale, -448, 448)) with
        the fp32 quotient correctly rounded, so later tokens of a block whose
        values exceed 448 * scale saturate.
    """
    codes = np.array(cache_codes, copy=True)
    sc = np.array(scales, dtype=np.float32, copy=True)
    x = np.asarray(new_values, dtype=np.float32)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    nb, hkv, bs, d = codes.shape
    if codes.dtype != np.uint8 or bs != block_size or x.shape != (slots.shape[0], hkv, d):
        raise ValueError("shape or dtype mismatch")
    live = [(t, int(s)) for t, s in enumerate(slots) if 0 <= s < nb * bs]
    if first_write:
        for t, s in live:
            if s % bs == 0:
                amax = np.abs(x[t]).max(axis=1)                                  # [Hkv], float32
                sc[s // bs] = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0))
    for t, s in live:
        q = x[t] / sc[s // bs][:, None]                                          # float32 quotient
        q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
        codes[s // bs, :, s % bs, :] = encode_e4m3fn_rne(q.astype(np.float64))
    return codes, sc
