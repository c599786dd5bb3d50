"""Input recipe and host block pool (support code, no device)."""

import numpy as np
import pytest
import torch

from workloads import (WORKLOADS, BlockPool, PoolExhausted, build_layout, make_host_inputs,
                       scaled, fp8_quantize_blocks, quantize_blocks, POISON_FP8_CODE,
                       POISON_INT8_CODE)
from oracle import decode_e4m3fn

BS = 16


def test_pool_allocates_in_free_order_and_recycles():
    p = BlockPool(4, [2, 0, 3, 1])
    assert [p.allocate() for _ in range(4)] == [2, 0, 3, 1]
    with pytest.raises(PoolExhausted):
        p.allocate()
    p.release(3)
    assert p.allocate() == 3
    with pytest.raises(ValueError):
        BlockPool(3, [0, 0, 1])


def test_pool_refcount_fork_and_free():
    p = BlockPool(8, range(8))
    p.new_sequence(0)
    for _ in range(40):
        p.append_token(0)
    p.fork(0, 1, 32)
    p.fork(0, 2, 32)
    assert p.refcount[:3] == [3, 3, 1]
    p.free_sequence(0)
    assert p.refcount[:3] == [2, 2, 0] and p.num_free == 6
    with pytest.raises(ValueError):
        p.fork(1, 3, 20)                    # not whole blocks
    with pytest.raises(NotImplementedError):
        q = BlockPool(4, range(4)); q.new_sequence(0)
        for _ in range(8):
            q.append_token(0)
        q.fork(0, 1, 16); q.num_tokens[1] = 8; q.tables[1] = q.tables[0][:1]
        q.tables[0] = q.tables[0][:1]; q.num_tokens[0] = 8; q.append_token(0)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_layout_shapes(name):
    w = WORKLOADS[name]
    if name.startswith("long_"):
        w = scaled(w, num_seqs=2, len_range=(4096, 4096))
    lay = build_layout(w)
    nblk = -(-lay.context_lens // BS)
    assert lay.block_tables.shape == (w.num_seqs, nblk.max())
    for b in range(w.num_seqs):
        row = lay.block_tables[b]
        assert (row[: nblk[b]] >= 0).all() and (row[nblk[b]:] == -1).all()
    used = lay.block_tables[lay.block_tables >= 0]
    counts = np.bincount(used, minlength=lay.num_blocks)
    assert np.array_equal(counts, lay.refcount)
    if w.shared_prefix_tokens:
        pb = w.shared_prefix_tokens // BS
        assert (lay.block_tables[:, :pb] == lay.block_tables[0, :pb]).all()
        assert (lay.refcount[lay.block_tables[0, :pb]] == w.num_seqs).all()
        assert counts.max() == w.num_seqs
    else:
        assert counts.max() == 1
    if w.append:
        # history + the appended slot = every position < L
        assert lay.history_mask.sum() == lay.context_lens.sum() - w.num_seqs - (
            (w.num_seqs - 1) * w.shared_prefix_tokens)
        for b in range(w.num_seqs):
            s = lay.slot_mapping[b]
            assert not lay.history_mask[s // BS, s % BS]
            assert s == lay.seq_slots[b][-1]


def test_published_shapes():
    w = WORKLOADS
    assert build_layout(w["tiny_f32"]).num_blocks == 64
    lay = build_layout(w["mha13b_prefix_f16"])
    assert lay.refcount.max() == 64 and (lay.refcount == 64).sum() == 75
    suf = lay.context_lens - 1200
    assert suf.min() >= 50 and suf.max() <= 400
    lay = build_layout(w["llama3_8b_bf16"])
    assert lay.context_lens.min() >= 512 and lay.context_lens.max() <= 8192
    assert lay.num_blocks == (-(-lay.context_lens // BS)).sum()


def test_host_inputs_poison_and_dtypes():
    lay = build_layout(WORKLOADS["tiny_f32"])
    x = make_host_inputs(lay)
    kc = x["k_cache"][0].numpy()
    hist = lay.history_mask
    assert np.isfinite(kc.transpose(0, 2, 1, 3)[hist]).all()
    assert np.isnan(kc.transpose(0, 2, 1, 3)[~hist]).all()
    assert x["q"].shape == (1, 4, 8, 64) and x["k_new"].shape == (1, 4, 2, 64)
    # same seed, same data
    y = make_host_inputs(lay)
    assert torch.equal(x["q"], y["q"]) and torch.equal(x["k_new"], y["k_new"])


def test_fp8_quantisation_recipe():
    w = scaled(WORKLOADS["long_fp8"], num_seqs=2, len_range=(64, 64))
    lay = build_layout(w)
    x = make_host_inputs(lay)
    codes = x["k_cache"][0].numpy()
    scales = x["k_scales"][0].numpy()
    vals = decode_e4m3fn(codes)
    hist = lay.history_mask
    assert not np.isnan(vals.transpose(0, 2, 1, 3)[hist]).any()
    # every tile's history reaches +-448 exactly once scaled: amax code is 0x7E/0xFE
    for blk in range(lay.num_blocks):
        for h in range(w.num_kv_heads):
            assert np.abs(vals[blk, h][hist[blk]]).max() == 448.0
            assert scales[blk, h] > 0
    # the slot the new token goes to is poisoned until the step quantises it
    s = lay.slot_mapping[0]
    assert (codes[s // 16, :, s % 16, :] == POISON_FP8_CODE).all()
    assert x["k_new"].dtype == torch.bfloat16
    assert x["q"].dtype == torch.bfloat16


def test_fp8_quantise_zero_tile_scale_is_one():
    x = torch.zeros((1, 1, BS, 4))
    codes, s = fp8_quantize_blocks(x)
    assert s.item() == 1.0 and (codes == 0).all()


def test_mixed_and_int8_recipes():
    """K fp8 / V int8, and int8 K with outlier channels: the codes, scales,
    poison and channel factors the recipe states."""
    w = scaled(WORKLOADS["long_fp8k_int8v"], num_seqs=2, len_range=(64, 64))
    lay = build_layout(w)
    x = make_host_inputs(lay)
    hist = lay.history_mask
    assert x["k_cache"].dtype == torch.uint8 and x["v_cache"].dtype == torch.int8
    v = x["v_cache"][0].numpy().transpose(0, 2, 1, 3)
    assert (np.abs(v[hist].astype(int)).max(axis=-1) <= 127).all()
    assert (v[~hist] == POISON_INT8_CODE).all()
    # every (block, head) tile's history reaches +-127
    vt = x["v_cache"][0].numpy()
    for blk in range(lay.num_blocks):
        assert (np.abs(vt[blk][:, hist[blk]].astype(int)).max(axis=(1, 2)) == 127).all()
    assert "k_channel_scales" not in x

    w = scaled(WORKLOADS["long_int8_kchan"], num_seqs=2, len_range=(64, 64))
    lay = build_layout(w)
    x = make_host_inputs(lay)
    c = x["k_channel_scales"].numpy()
    assert c.shape == (w.num_kv_heads, w.head_dim)
    assert ((c == 16).sum(axis=1) == w.k_outliers).all() and ((c == 1) | (c == 16)).all()
    # the new token carries the outliers: its outlier channels are ~16x larger
    kn = x["k_new"][0].float().numpy()
    for h in range(w.num_kv_heads):
        ratio = np.abs(kn[:, h, c[h] == 16]).mean() / np.abs(kn[:, h, c[h] == 1]).mean()
        assert 4 < ratio < 64
    # int8 rounding of the recipe: halves to even
    codes, s = quantize_blocks(torch.tensor([0.5, 1.5, 2.5, -0.5, 127.0]).view(1, 1, 1, 5),
                               code="int8")
    assert s.item() == 1.0 and codes.flatten().tolist() == [0, 2, 2, 0, 127]


def test_full_precision_sink_recipe():
    """Side tiles hold positions < S in q's dtype (x4 draws), the rest of each
    tile is NaN, and the cache slots of those positions are poisoned."""
    w = scaled(WORKLOADS["long_fp8k_int8v"], num_seqs=3, len_range=(3, 40), fp_sinks=5, num_layers=2)
    lay = build_layout(w)
    x = make_host_inputs(lay)
    S = 5
    order = x["sink_tiles_of_seq"].numpy()
    assert sorted(order.tolist()) == [0, 1, 2]
    for layer in range(2):
        for b in range(3):
            t = x["sink_k"][layer][order[b]].float().numpy()          # [Hkv, 16, D]
            assert np.isfinite(t[:, :S]).all() and np.isnan(t[:, S:]).all()
            assert np.abs(t[:, :S]).std() > 2
            for pos, slot in enumerate(lay.seq_slots[b][:S]):
                slot = int(slot)
                assert (x["k_cache"][layer][slot // 16, :, slot % 16] == POISON_FP8_CODE).all()
                assert (x["v_cache"][layer][slot // 16, :, slot % 16] == POISON_INT8_CODE).all()
    pos = lay.context_lens - 1
    side = x["sink_slot_mapping"].numpy()
    for b in range(3):
        assert side[b] == (order[b] * 16 + pos[b] if pos[b] < S else -1)
