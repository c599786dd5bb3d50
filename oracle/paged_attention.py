"""Single-query decode attention over a paged KV cache, in float64.

What is computed, and where the pages state it:
  * [P5] section 4 (block table): a sequence's tokens live in
    fixed blocks of `block_size` tokens; its block table lists the physical
    block of each logical block, so logical position `pos` is found in block
    table[pos // block_size] at offset pos % block_size.
  * [P1] section 4.3: the attention kernel fetches K and V through the block
    table from non-contiguous places; paging changes where bytes live, not
    what is computed.
  * [P1] section 2.1: attention is softmax(Q K^T / sqrt(d_head)) V; here the
    scale is an argument (1/sqrt(head_dim) in every workload).
  * [P1] section 2.2: at a decode step the single new query attends to the
    keys of every cached position, the new token's own included.
  * [P5] section 2 and [P3] section 3.3: with grouped-query attention every g
    consecutive query heads share one K/V head (g = Hq / Hkv; MQA is Hkv = 1).
  * [P5] section 7: quantised K/V carry one scale per head; here one fp32
    scale per (physical block, KV head), and the value used is code * scale.
    [P1] section 5.2 names finer granularities against K's outlier
    channels: per channel (below) or per token -- one fp32 scale per
    (slot, KV head) -- and quantising V alone with K kept in 16 bits.
  * [P5] section 7: K is the more sensitive of the two, so K may stay in FP8
    while V goes to INT8 (symmetric integer codes, value = code * scale);
    [P1] section 5.2: K has outlier channels, which per-channel scaling
    absorbs -- here an optional fp32 factor per (KV head, channel) applied on
    top of the per-(block, head) scale.
  * [P1] section 5.3: with a sliding window of W, a position attends only to
    the most recent W tokens (itself included), optionally together with the
    first few tokens of the sequence (attention sinks), which [P1] 5.3 and
    [P5] section 7 single out as tokens that must not be dropped; [P5]
    section 7 also keeps them in their original precision when the rest of
    the cache is quantised (optional full-precision side tiles here).

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .values import stored_to_f64


def page_of(table_row, pos, block_size):
    """Where logical position(s) `pos` of a sequence are stored: the paging
    definition splits a position into (logical page, offset in the page) and
    the sequence's table maps the logical page to a physical one.
    Returns (physical pages, offsets)."""
    logical_page, offset = np.divmod(np.asarray(pos), int(block_size))
    return np.asarray(table_row)[logical_page], offset


def attended_positions(length: int, window: int = 0, sinks: int = 0) -> np.ndarray:
    """Positions the query of a sequence of `length` tokens attends to.

    window = 0: all of them.  window > 0: the last `window` positions, plus
    the first `sinks` positions (sinks only matter together with a window).
    """
    L = int(length)
    if window <= 0:
        return np.arange(L)
    recent = np.arange(max(0, L - int(window)), L)
    first = np.arange(min(int(sinks), L))
    return np.union1d(first, recent)


QUANTISED = ("fp8_e4m3", "int8")


def gather_sequence(cache, table_row, length: int, kv_tag: str, kv_heads=None,
                    scales=None, block_size: int = 16, positions=None,
                    channel_scales=None) -> np.ndarray:
    """Contiguous float64 [n, len(kv_heads), D] copy of one sequence's tokens.

    `cache` is the raw storage array [num_blocks, Hkv, block_size, D] (uint16
    bits for bf16, uint8 codes for fp8, int8 codes for int8); `scales` is
    required for the quantised tags: fp32 [num_blocks, Hkv], one scale that
    multiplies every element of its (block, head) tile, or fp32
    [num_blocks, Hkv, block_size], one scale per (slot, head) -- the
    per-token granularity of [P1] section 5.2 -- that multiplies the D
    elements of that token's row; `channel_scales` ([Hkv, D] fp32,
    optional) multiplies channel d of head h.  The tokens are `positions`
    (default: 0 .. length-1), all < length.
    """
    nb = cache.shape[0]
    if kv_heads is None:
        kv_heads = np.arange(cache.shape[1])
    kv_heads = np.asarray(kv_heads)
    pos = np.arange(int(length)) if positions is None else np.asarray(positions, dtype=np.int64)
    if len(pos) and (pos.min() < 0 or pos.max() >= length):
        raise IndexError("position outside the sequence")
    blk, off = page_of(table_row, pos, block_size)
    if len(pos) and (blk.min() < 0 or blk.max() >= nb):
        raise IndexError("block table entry outside the pool for a position < length")
    raw = cache[blk[:, None], kv_heads[None, :], off[:, None], :]      # [L, h, D]
    vals = stored_to_f64(raw, kv_tag)
    if kv_tag in QUANTISED:
        if scales is None:
            raise ValueError("quantised caches need their per-(block, head) scales")
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)
        if s.shape == (nb, cache.shape[1]):
            vals = vals * s[blk[:, None], kv_heads[None, :]][:, :, None]
        elif s.shape == (nb, cache.shape[1], block_size):
            vals = vals * s[blk[:, None], kv_heads[None, :], off[:, None]][:, :, None]
        else:
            raise ValueError("scales must be [num_blocks, Hkv] or [num_blocks, Hkv, block_size]")
    elif scales is not None:
        raise ValueError("scales apply to quantised caches only")
    if channel_scales is not None:
        c = np.asarray(channel_scales, dtype=np.float32).astype(np.float64)
        vals = vals * c[kv_heads][None, :, :]
    return vals


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                           *, q_tag: str, kv_tag: str, k_scales=None, v_scales=None,
                           seqs: Optional[Sequence[int]] = None,
                           q_heads: Optional[Sequence[int]] = None,
                           block_size: int = 16, window: int = 0, sinks: int = 0,
                           v_tag: Optional[str] = None, k_channel_scales=None,
                           sink_k=None, sink_v=None, sink_blocks=None,
                           sink_tag: Optional[str] = None) -> np.ndarray:
    """out[b, i, :] for b in `seqs`, i in `q_heads` (all by default), float64.

    q: [B, Hq, D] storage array; caches: [num_blocks, Hkv, block_size, D];
    block_tables: int [B, max_blocks]; context_lens: int [B].  window/sinks
    restrict the attended positions (see attended_positions).  v_tag (default
    kv_tag) is the V cache's format when it differs from K's;
    k_channel_scales ([Hkv, D]) multiplies K's channels.

    Full-precision sinks ([P5] section 7: attention-sink tokens keep their
    original precision, since their magnitudes would spoil a shared scale):
    with sink_k/sink_v ([num_sink_tiles, Hkv, block_size, D] of sink_tag,
    default q_tag) and sink_blocks ([B]), position p < `sinks` of sequence b
    is read, as stored, from tile sink_blocks[b], offset p, instead of the
    cache; the attended positions are unchanged.
    """
    v_tag = kv_tag if v_tag is None else v_tag
    sink_tag = q_tag if sink_tag is None else sink_tag
    side = sink_k is not None
    if side and not (1 <= sinks <= block_size and sink_v is not None and sink_blocks is not None):
        raise ValueError("full-precision sinks need 1 <= sinks <= block_size, both tiles and sink_blocks")
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = Hq // Hkv
    seqs = list(range(B)) if seqs is None else list(seqs)
    q_heads = list(range(Hq)) if q_heads is None else list(q_heads)
    kv_for = [i // g for i in q_heads]
    kv_needed = sorted(set(kv_for))
    col = {h: c for c, h in enumerate(kv_needed)}
    out = np.zeros((len(seqs), len(q_heads), D), dtype=np.float64)
    qv = stored_to_f64(np.asarray(q)[seqs][:, q_heads], q_tag)       # [nb, nh, D]
    for r, b in enumerate(seqs):
        L = int(context_lens[b])
        pos = attended_positions(L, window, sinks)
        if len(pos) == 0:
            continue
        if side:
            first, pos = pos[pos < sinks], pos[pos >= sinks]
        K = gather_sequence(k_cache, block_tables[b], L, kv_tag, kv_needed, k_scales, block_size, pos,
                            k_channel_scales)
        V = gather_sequence(v_cache, block_tables[b], L, v_tag, kv_needed, v_scales, block_size, pos)
        if side and len(first):
            tile = int(sink_blocks[b])
            sk = np.asarray(sink_k)[tile][kv_needed][:, first, :].transpose(1, 0, 2)   # [n, h, D]
            sv = np.asarray(sink_v)[tile][kv_needed][:, first, :].transpose(1, 0, 2)
            K = np.concatenate([stored_to_f64(sk, sink_tag), K])
            V = np.concatenate([stored_to_f64(sv, sink_tag), V])
        for c, i in enumerate(q_heads):
            h = col[kv_for[c]]
            s = scale * (K[:, h, :] @ qv[r, c])          # [L] scores
            w = np.exp(s - s.max())                       # softmax numerator
            out[r, c] = (w @ V[:, h, :]) / w.sum()
    return out
