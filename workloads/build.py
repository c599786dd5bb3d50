"""Build block tables and seeded K/V/q tensors for a decode workload.

Recipe (all seeded from the workload's seed):
  * lengths: explicit, or uniform integers in the stated range (for a shared
    prefix the range is that of the private suffix, added to the prefix);
  * physical pool: `num_blocks` (or exactly what the batch needs); the free
    list is a seeded random permutation of the block ids, so consecutive
    logical blocks of a sequence land on scattered physical blocks;
  * tables: sequence 0 takes its prefix blocks, the other sequences fork them
    (reference count = number of sequences), then every sequence takes fresh
    blocks for its private history, then the decode step reserves the slot of
    each sequence's new token (a new block when the last one is full);
  * values: q, K, V ~ N(0, 1) drawn in fp32 and rounded to the storage dtype;
    every cache slot that holds no history token (block tails, unused blocks,
    the slot the new token will be written to) is poisoned with NaN (float
    caches) or the e4m3 NaN code 0x7F (fp8 caches), so a read of it shows up;
  * 8-bit caches: per (block, kv_head) tile, scale = amax|x| / QMAX in fp32
    (1.0 for an all-zero tile; QMAX 448 for fp8 e4m3, 127 for int8) over the
    tile's history tokens, code = round-to-nearest-even(x / scale) clamped to
    +-QMAX, done by torch (float8_e4m3fn cast, or round then int8); poisoned
    slots hold 0x7F (fp8 NaN) or -128 (the unused int8 code); the new token's
    K/V are drawn in the query dtype and quantised on write, with its block's
    existing scale, by the step itself;
  * per-token scales (k_scale_tok / v_scale_tok): the same, with one scale
    per (slot, kv_head), amax|x| / QMAX over that token's row; a slot that
    holds no token has a NaN scale (poisoned like its codes); the new
    token sets its own slot's scale when it is written;
  * a 16-bit K with an 8-bit V (kv_dtype f16/bf16, v_dtype fp8/int8): K is
    drawn as for a 16-bit cache, V quantised as above;
  * K outlier channels (k_outliers > 0): in each KV head that many channels,
    chosen at random, are 16x larger, in the history and in the new token
    alike; K then has per-channel factors c[h][d] (16 on those channels, 1
    elsewhere) that every K value is divided by before quantising;
  * shared-prefix groups: a shared prefix makes one group of all sequences
    (group_starts [0, B], group_blocks [prefix / 16]); share_prefixes()
    rewrites a layout's tables into several groups, each member pointing
    its first blocks at those of the group's first sequence, and releases
    (poisons) the blocks that were replaced;
  * full-precision sinks (fp_sinks = S > 0): sequence b's first S positions
    live in side tile sink_tiles_of_seq[b] (a seeded permutation of the B
    tiles), in q's dtype, drawn N(0, 1) x 4 (sink tokens stand apart in
    magnitude); the rest of each tile, and the cache slots of those
    positions, are poisoned; a new token at a position < S goes to its tile
    (sink_slot_mapping = tile * 16 + position, else -1).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from .pool import BlockPool
from .specs import DecodeWorkload

POISON_FP8_CODE = 0x7F
POISON_INT8_CODE = -128
FP8_MAX = 448.0
INT8_MAX = 127.0
OUTLIER_GAIN = 16.0

_TORCH_DTYPE = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8_e4m3": torch.uint8,
    "int8": torch.int8,
}
_QMAX = {"fp8_e4m3": FP8_MAX, "int8": INT8_MAX}
_POISON = {"fp8_e4m3": POISON_FP8_CODE, "int8": POISON_INT8_CODE}


def torch_dtype(tag: str) -> torch.dtype:
    return _TORCH_DTYPE[tag]


@dataclass
class DecodeLayout:
    spec: DecodeWorkload
    context_lens: np.ndarray        # int32 [B], post-append
    block_tables: np.ndarray        # int32 [B, max_blocks], -1 padded
    num_blocks: int
    slot_mapping: Optional[np.ndarray]  # int64 [B] slot of the new token, or None
    history_mask: np.ndarray        # bool [num_blocks, block_size]: slot holds a history token
    refcount: np.ndarray            # int32 [num_blocks]
    seq_slots: list                 # per sequence: int64 [L] flat slot of every position,
                                    # in the order the pool handed them out
    # shared-prefix groups: group g is the sequences [group_starts[g],
    # group_starts[g + 1]), whose first group_blocks[g] table entries are the
    # same physical blocks (None: no groups)
    group_starts: Optional[np.ndarray] = None   # int32 [G + 1]
    group_blocks: Optional[np.ndarray] = None   # int32 [G]

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


def _lengths(spec: DecodeWorkload, rng: np.random.Generator) -> np.ndarray:
    if spec.context_lens is not None:
        lens = np.asarray(spec.context_lens, dtype=np.int64)
        if lens.shape[0] != spec.num_seqs:
            raise ValueError("context_lens does not match num_seqs")
    else:
        lo, hi = spec.len_range
        lens = rng.integers(lo, hi + 1, size=spec.num_seqs, dtype=np.int64)
        lens = lens + spec.shared_prefix_tokens
    return lens


def _blocks_needed(spec: DecodeWorkload, lens: np.ndarray) -> int:
    bs = spec.block_size
    p = spec.shared_prefix_tokens
    if p:
        return p // bs + int(sum(-(-(int(L) - p) // bs) for L in lens))
    return int(sum(-(-int(L) // bs) for L in lens))


def build_layout(spec: DecodeWorkload) -> DecodeLayout:
    bs = spec.block_size
    rng = np.random.default_rng(spec.seed)
    lens = _lengths(spec, rng)
    if spec.shared_prefix_tokens % bs:
        raise ValueError("a shared prefix must be whole blocks")
    if spec.shared_prefix_tokens and int(lens.min()) <= spec.shared_prefix_tokens:
        raise ValueError("every sequence must extend past the shared prefix")
    need = _blocks_needed(spec, lens)
    nb = spec.num_blocks if spec.num_blocks is not None else need
    if nb < need:
        raise ValueError(f"pool of {nb} blocks is smaller than the {need} needed")
    pool = BlockPool(nb, rng.permutation(nb), block_size=bs)

    hist = lens - 1 if spec.append else lens.copy()
    history_mask = np.zeros((nb, bs), dtype=bool)

    seq_slots = {b: [] for b in range(spec.num_seqs)}

    def take(seq: int, count: int) -> None:
        for _ in range(count):
            slot = pool.append_token(seq)
            seq_slots[seq].append(slot)
            history_mask[slot // bs, slot % bs] = True

    p = spec.shared_prefix_tokens
    B = spec.num_seqs
    pool.new_sequence(0)
    if p:
        take(0, p)
        for b in range(1, B):
            pool.fork(0, b, p)
            seq_slots[b] = list(seq_slots[0][:p])
    else:
        for b in range(1, B):
            pool.new_sequence(b)
    for b in range(B):
        take(b, int(hist[b]) - pool.num_tokens[b])

    slot_mapping = None
    if spec.append:
        slot_mapping = np.array([pool.append_token(b) for b in range(B)], dtype=np.int64)
        for b in range(B):
            seq_slots[b].append(int(slot_mapping[b]))

    max_blocks = max(len(pool.tables[b]) for b in range(B))
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    for b in range(B):
        t = pool.tables[b]
        tables[b, : len(t)] = t
    return DecodeLayout(
        spec=spec,
        context_lens=lens.astype(np.int32),
        block_tables=tables,
        num_blocks=nb,
        slot_mapping=slot_mapping,
        history_mask=history_mask,
        refcount=np.asarray(pool.refcount, dtype=np.int32),
        seq_slots=[np.asarray(seq_slots[b], dtype=np.int64) for b in range(B)],
        group_starts=np.array([0, B], dtype=np.int32) if p else None,
        group_blocks=np.array([p // bs], dtype=np.int32) if p else None,
    )


def share_prefixes(layout: DecodeLayout, starts, blocks) -> DecodeLayout:
    """A copy of `layout` in which the sequences of group g = [starts[g],
    starts[g + 1]) all point their first blocks[g] table entries at the
    blocks of the group's first sequence (a fork of that sequence's prefix).

    The blocks the other members held there are released: no longer
    history, so the tensors poison them.  Every member must keep at least
    one private history position past the shared blocks (the new token then
    never lands in a shared block).
    """
    bs = layout.spec.block_size
    starts = np.asarray(starts, dtype=np.int32)
    blocks = np.asarray(blocks, dtype=np.int32)
    if starts.shape != (blocks.shape[0] + 1,) or (np.diff(starts) < 0).any():
        raise ValueError("starts must be nondecreasing [G + 1], blocks [G]")
    tables = layout.block_tables.copy()
    mask = layout.history_mask.copy()
    ref = layout.refcount.copy()
    slots = [s.copy() for s in layout.seq_slots]
    hist = layout.context_lens.astype(np.int64) - (1 if layout.slot_mapping is not None else 0)
    for g in range(blocks.shape[0]):
        s0, s1, n = int(starts[g]), int(starts[g + 1]), int(blocks[g])
        for b in range(s0 + 1, s1):
            if hist[b] <= n * bs or hist[s0] <= n * bs:
                raise ValueError("a group member would not extend past the shared blocks")
            for j in range(n):
                old, new = int(tables[b, j]), int(tables[s0, j])
                if old == new:
                    continue
                ref[old] -= 1
                if ref[old] == 0:
                    mask[old] = False
                ref[new] += 1
                tables[b, j] = new
            slots[b][: n * bs] = slots[s0][: n * bs]
    return DecodeLayout(spec=layout.spec, context_lens=layout.context_lens, block_tables=tables,
                        num_blocks=layout.num_blocks, slot_mapping=layout.slot_mapping,
                        history_mask=mask, refcount=ref, seq_slots=slots,
                        group_starts=starts, group_blocks=blocks)


# ---------------------------------------------------------------------------
# tensors
# ---------------------------------------------------------------------------

def quantize_blocks(x: torch.Tensor, valid: Optional[torch.Tensor] = None, code: str = "fp8_e4m3"):
    """x: fp32 [NB, H, bs, D] -> (codes same shape, scales fp32 [NB, H]).

    The scale of each (block, head) tile is its amax over valid slots / QMAX;
    codes are uint8 e4m3fn bits or int8 integers.
    """
    qmax = _QMAX[code]
    if valid is not None:
        xm = x.masked_fill(~valid.view(valid.shape[0], 1, valid.shape[1], 1), 0.0)
    else:
        xm = x
    amax = xm.abs().amax(dim=(2, 3))
    scales = torch.where(amax > 0, amax / qmax, torch.ones_like(amax)).to(torch.float32)
    y = (x / scales[:, :, None, None]).clamp_(-qmax, qmax)
    if code == "fp8_e4m3":
        return y.to(torch.float8_e4m3fn).view(torch.uint8), scales
    return torch.round(y).to(torch.int8), scales          # round: halves to even


def quantize_tokens(x: torch.Tensor, code: str = "fp8_e4m3"):
    """x: fp32 [NB, H, bs, D] -> (codes same shape, scales fp32 [NB, H, bs]):
    one scale per (slot, head), the row's amax / QMAX (1.0 for a zero row)."""
    qmax = _QMAX[code]
    amax = x.abs().amax(dim=3)
    scales = torch.where(amax > 0, amax / qmax, torch.ones_like(amax)).to(torch.float32)
    y = (x / scales[..., None]).clamp_(-qmax, qmax)
    if code == "fp8_e4m3":
        return y.to(torch.float8_e4m3fn).view(torch.uint8), scales
    return torch.round(y).to(torch.int8), scales          # round: halves to even


def fp8_quantize_blocks(x: torch.Tensor, valid: Optional[torch.Tensor] = None):
    return quantize_blocks(x, valid, "fp8_e4m3")


def outlier_factors(spec: DecodeWorkload, device: str) -> Optional[torch.Tensor]:
    """fp32 [Hkv, D]: OUTLIER_GAIN on spec.k_outliers seeded channels per head, else 1."""
    if not spec.k_outliers:
        return None
    rng = np.random.default_rng(spec.seed + 7919)
    c = np.ones((spec.num_kv_heads, spec.head_dim), np.float32)
    for h in range(spec.num_kv_heads):
        c[h, rng.choice(spec.head_dim, spec.k_outliers, replace=False)] = OUTLIER_GAIN
    return torch.from_numpy(c).to(device)


def _gen(device: str, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, gen, device, dtype_tag):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if dtype_tag == "fp8_e4m3":
        return x
    return x.to(torch_dtype(dtype_tag))


def _make_inputs(layout: DecodeLayout, device: str, layers: Optional[int]) -> Dict[str, torch.Tensor]:
    spec = layout.spec
    nl = spec.num_layers if layers is None else layers
    B, Hq, Hkv, D, bs = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    NB = layout.num_blocks
    gen = _gen(device, spec.seed)
    valid = torch.from_numpy(layout.history_mask).to(device)
    poison = ~valid.view(NB, 1, bs, 1)
    tags = {"k": spec.kv_dtype, "v": spec.v_tag}
    chan = outlier_factors(spec, device)
    out: Dict[str, torch.Tensor] = {}
    out["q"] = _normal((nl, B, Hq, D), gen, device, spec.q_dtype)
    k_cache = torch.empty((nl, NB, Hkv, bs, D), dtype=torch_dtype(tags["k"]), device=device)
    v_cache = torch.empty((nl, NB, Hkv, bs, D), dtype=torch_dtype(tags["v"]), device=device)
    scales = {}
    for name, cache in (("k", k_cache), ("v", v_cache)):
        tag = tags[name]
        if tag in _QMAX:
            tok = spec.k_scale_tok if name == "k" else spec.v_scale_tok
            sc = torch.empty((nl, NB, Hkv) + ((bs,) if tok else ()), dtype=torch.float32, device=device)
            for layer in range(nl):
                x = torch.randn((NB, Hkv, bs, D), generator=gen, device=device, dtype=torch.float32)
                # with outlier channels x is already K / c: the history's K is
                # code * scale * c, its outliers carried by c
                codes, s = quantize_tokens(x, tag) if tok else quantize_blocks(x, valid, tag)
                del x
                codes.masked_fill_(poison, _POISON[tag])
                if tok:                       # a slot with no token has no scale either
                    s.masked_fill_(~valid.view(NB, 1, bs), float("nan"))
                cache[layer].copy_(codes)
                sc[layer].copy_(s)
                del codes
            scales[name] = sc
        else:
            for layer in range(nl):
                x = torch.randn((NB, Hkv, bs, D), generator=gen, device=device, dtype=torch.float32)
                cache[layer].copy_(x)        # rounds to the storage dtype (RNE)
                del x
                cache[layer].masked_fill_(poison, float("nan"))
    out["k_cache"], out["v_cache"] = k_cache, v_cache
    for name in ("k", "v"):
        if name in scales:
            out[f"{name}_scales"] = scales[name]
    if chan is not None:
        out["k_channel_scales"] = chan
    if spec.fp_sinks:
        S = spec.fp_sinks
        if not (spec.quantised and 1 <= S <= bs):
            raise ValueError("full-precision sinks need an 8-bit cache and 1..16 positions")
        order = torch.from_numpy(np.random.default_rng(spec.seed + 104729).permutation(B).astype(np.int32))
        qdt = torch_dtype(spec.q_dtype)
        tiles = {}
        for name in ("k", "v"):
            t = torch.full((nl, B, Hkv, bs, D), float("nan"), dtype=qdt, device=device)
            for layer in range(nl):
                x = torch.randn((B, Hkv, S, D), generator=gen, device=device, dtype=torch.float32) * 4
                t[layer][order.to(device).long(), :, :S, :] = x.to(qdt)
            tiles[name] = t
        out["sink_k"], out["sink_v"] = tiles["k"], tiles["v"]
        out["sink_tiles_of_seq"] = order.to(device)
        # the cache never serves these positions: poison them there
        for b in range(B):
            for slot in layout.seq_slots[b][:S]:
                slot = int(slot)
                for name, cache in (("k", k_cache), ("v", v_cache)):
                    cache[:, slot // bs, :, slot % bs, :] = _POISON[tags[name]]
        if spec.append:
            pos = layout.context_lens.astype(np.int64) - 1
            side = np.where(pos < S, order.numpy().astype(np.int64) * bs + pos, -1)
            out["sink_slot_mapping"] = torch.from_numpy(side).to(device)
    if spec.append:
        # 8-bit caches quantise the new token on write; its K/V arrive in the
        # query's dtype
        src_tag = spec.q_dtype if spec.quantised else spec.kv_dtype
        out["k_new"] = _normal((nl, B, Hkv, D), gen, device, src_tag)
        out["v_new"] = _normal((nl, B, Hkv, D), gen, device, src_tag)
        if chan is not None:
            out["k_new"] = (out["k_new"].float() * chan).to(out["k_new"].dtype)
        out["slot_mapping"] = torch.from_numpy(layout.slot_mapping).to(device)
    out["block_tables"] = torch.from_numpy(layout.block_tables).to(device)
    out["context_lens"] = torch.from_numpy(layout.context_lens).to(device)
    if layout.group_starts is not None:
        out["group_starts"] = torch.from_numpy(layout.group_starts).to(device)
        out["group_blocks"] = torch.from_numpy(layout.group_blocks).to(device)
    return out


def make_host_inputs(layout: DecodeLayout, layers: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """All tensors on the CPU (small workloads; the oracle reads these)."""
    return _make_inputs(layout, "cpu", layers)


def make_device_inputs(layout: DecodeLayout, device: str = "cuda", layers: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """All tensors drawn directly on `device` (full-size workloads)."""
    return _make_inputs(layout, device, layers)
