"""Per-step K/V append into a paged cache, on raw bits.

[P1] section 2.3: each decode step writes the new token's K and V at the
sequence's current length and then advances the length by one.  [P5]
section 4 (block tables): with paging the write goes to the flat slot
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


QMAX = {"fp8_e4m3": E4M3_MAX, "int8": 127.0}
CODE_DTYPE = {"fp8_e4m3": np.uint8, "int8": np.int8}


def _encode(q: np.ndarray, code: str) -> np.ndarray:
    """fp32 quotients already clamped to +-QMAX -> codes."""
    if code == "fp8_e4m3":
        return encode_e4m3fn_rne(q.astype(np.float64))
    r = np.rint(np.where(np.isnan(q), np.float32(0), q))    # rint: halves to even; NaN -> 0
    return r.astype(np.int8)


def kv_append_quant(cache_codes, scales, new_values, slot_mapping, *, code: str,
                    first_write: bool, channel_scales=None, block_size: int = 16,
                    granularity: str = "block"):
    """Quantise-on-write into an 8-bit cache; returns new (codes, scales).

    [P5] section 7: 8-bit K/V with one scale per head, and K in FP8 with V in
    INT8 as the mixed form; [P1] section 5.2: per-channel factors for K's
    outlier channels, or per-token scales.  `code` is "fp8_e4m3" (OCP
    e4m3fn, QMAX = 448) or "int8" (symmetric, QMAX = 127, -128 unused).

    granularity "token": scales is float32 [NB, Hkv, bs], one per (slot,
    head), and every written token sets its own scales from its own row
    before its codes are taken -- scale = float32(max_d |y[t, h, d]|) /
    float32(QMAX) in fp32 (1.0 when that max is 0) -- so no value
    saturates; `first_write` must then be False (it has no meaning).  The
    rest of this docstring describes the default, granularity "block".

    cache_codes: [NB, Hkv, bs, D] codes; scales: float32 [NB, Hkv];
    new_values: float32 [T, Hkv, D] (the source values, widened exactly);
    channel_scales: optional float32 [Hkv, D].
    For every token t with slot s = slot_mapping[t] in [0, NB * bs):
      * y = float32(x) / float32(channel_scales[h, d]) (a correctly rounded
        fp32 division), or x itself without channel scales;
      * first_write and s % bs == 0 (the block's first token): the block's
        scale for head h becomes float32(max_d |y[t, h, d]|) / float32(QMAX)
        in fp32 (1.0 when that max is 0); all such scales are set before any
        token is quantised;
      * every element becomes the nearest code (ties to even) of
        clamp(float32(y) / scale, -QMAX, QMAX), the fp32 quotient correctly
        rounded, so later tokens of a block whose values exceed QMAX * scale
        saturate.  NaN stays NaN in fp8 and becomes 0 in int8.
    """
    qmax = np.float32(QMAX[code])
    codes = np.array(cache_codes, copy=True)
    sc = np.array(scales, dtype=np.float32, copy=True)
    x = np.asarray(new_values, dtype=np.float32)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    nb, hkv, bs, d = codes.shape
    if codes.dtype != CODE_DTYPE[code] or bs != block_size or x.shape != (slots.shape[0], hkv, d):
        raise ValueError("shape or dtype mismatch")
    if channel_scales is not None:
        c = np.asarray(channel_scales, dtype=np.float32)
        if c.shape != (hkv, d):
            raise ValueError("channel scales must be [Hkv, D]")
        x = x / c[None, :, :]                                                    # float32 quotient
    live = [(t, int(s)) for t, s in enumerate(slots) if 0 <= s < nb * bs]
    if granularity == "token":
        if first_write or sc.shape != (nb, hkv, bs):
            raise ValueError("per-token scales are [NB, Hkv, bs] and always set by their token")
        for t, s in live:
            amax = np.abs(x[t]).max(axis=1)                                      # [Hkv], float32
            tok = np.where(amax > 0, amax / qmax, np.float32(1.0))
            sc[s // bs, :, s % bs] = tok
            q = np.clip(x[t] / tok[:, None], -qmax, qmax)                        # float32 quotient
            codes[s // bs, :, s % bs, :] = _encode(q, code)
        return codes, sc
    if granularity != "block" or sc.shape != (nb, hkv):
        raise ValueError("granularity is 'block' (scales [NB, Hkv]) or 'token' (scales [NB, Hkv, bs])")
    if first_write:
        for t, s in live:
            if s % bs == 0:
                amax = np.abs(x[t]).max(axis=1)                                  # [Hkv], float32
                sc[s // bs] = np.where(amax > 0, amax / qmax, np.float32(1.0))
    for t, s in live:
        q = x[t] / sc[s // bs][:, None]                                          # float32 quotient
        q = np.clip(q, -qmax, qmax)
        codes[s // bs, :, s % bs, :] = _encode(q, code)
    return codes, sc


def kv_append_fp8(cache_codes, scales, new_values, slot_mapping, *, first_write: bool,
                  block_size: int = 16, channel_scales=None):
    """kv_append_quant into an e4m3fn cache (QMAX 448)."""
    return kv_append_quant(cache_codes, scales, new_values, slot_mapping, code="fp8_e4m3",
                           first_write=first_write, channel_scales=channel_scales,
                           block_size=block_size)


def kv_append_int8(cache_codes, scales, new_values, slot_mapping, *, first_write: bool,
                   block_size: int = 16, channel_scales=None):
    """kv_append_quant into a symmetric int8 cache (QMAX 127)."""
    return kv_append_quant(cache_codes, scales, new_values, slot_mapping, code="int8",
                           first_write=first_write, channel_scales=channel_scales,
                           block_size=block_size)
