"""Pins for the float64 paged decode attention oracle.

Nothing here retypes the oracle's formula.  The oracle is checked against
  * torch's scaled_dot_product_attention in float64 on contiguous K/V whose
    paged copy was laid down token by token by the block pool (so the pool's
    incremental bookkeeping, not the oracle's page_of(), decides where a token
    lives);
  * closed forms (constant V, zero query, one token, one dominant key);
  * invariances (physical block permutation, GQA vs K/V heads duplicated,
    shared prefix vs private copies, storage dtype decoded by torch);
and a set of planted mistakes must each be caught by at least one pin.
"""

import math
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import paged_decode_attention, page_of
from workloads import BlockPool, build_layout, make_host_inputs, WORKLOADS, scaled

BS = 16


# --------------------------------------------------------------------------
# builders that do not use the oracle
# --------------------------------------------------------------------------

def paged_from_contiguous(seq_k, seq_v, num_blocks, seed, storage=np.float64, fill=np.nan,
                          shared_prefix=0):
    """Lay contiguous per-sequence K/V ([L, H, D] each) into a paged pool.

    Tokens are appended one at a time through BlockPool; the slot it returns
    is where the token is written.  Returns (k_cache, v_cache, tables, lens).
    """
    B = len(seq_k)
    H, D = seq_k[0].shape[1:]
    rng = np.random.default_rng(seed)
    pool = BlockPool(num_blocks, rng.permutation(num_blocks), BS)
    kc = np.full((num_blocks, H, BS, D), fill, dtype=storage)
    vc = np.full_like(kc, fill)

    def put(b, pos, slot):
        kc[slot // BS, :, slot % BS, :] = seq_k[b][pos]
        vc[slot // BS, :, slot % BS, :] = seq_v[b][pos]

    pool.new_sequence(0)
    if shared_prefix:
        for pos in range(shared_prefix):
            put(0, pos, pool.append_token(0))
        for b in range(1, B):
            pool.fork(0, b, shared_prefix)
    else:
        for b in range(1, B):
            pool.new_sequence(b)
    for b in range(B):
        for pos in range(pool.num_tokens[b], len(seq_k[b])):
            put(b, pos, pool.append_token(b))
    maxb = max(1, max(len(pool.tables[b]) for b in range(B)))
    tables = np.full((B, maxb), -1, dtype=np.int32)
    for b in range(B):
        tables[b, : len(pool.tables[b])] = pool.tables[b]
    lens = np.array([len(k) for k in seq_k], dtype=np.int32)
    return kc, vc, tables, lens


def sdpa_reference(q, seq_k, seq_v, scale):
    """float64 torch SDPA per sequence; K/V heads repeated g times."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = seq_k[b].shape[0]
        if L == 0:
            continue
        g = Hq // seq_k[b].shape[1]
        K = torch.from_numpy(np.ascontiguousarray(seq_k[b])).permute(1, 0, 2).repeat_interleave(g, 0)
        V = torch.from_numpy(np.ascontiguousarray(seq_v[b])).permute(1, 0, 2).repeat_interleave(g, 0)
        qq = torch.from_numpy(np.ascontiguousarray(q[b]))[:, None, :]
        o = F.scaled_dot_product_attention(qq, K.contiguous(), V.contiguous(), scale=scale)
        out[b] = o[:, 0, :].numpy()
    return out


def random_case(rng, B, Hq, Hkv, D, lens):
    q = rng.standard_normal((B, Hq, D))
    seq_k = [rng.standard_normal((L, Hkv, D)) for L in lens]
    seq_v = [rng.standard_normal((L, Hkv, D)) for L in lens]
    return q, seq_k, seq_v


def run_oracle(mod, q, kc, vc, tables, lens, scale, q_tag="f32", kv_tag="f32", **kw):
    cast = {"f32": np.float32}
    if kv_tag == "f32":
        kc, vc = kc.astype(np.float32), vc.astype(np.float32)
    if q_tag == "f32":
        q = q.astype(np.float32)
    return mod.paged_decode_attention(q, kc, vc, tables, lens, scale, q_tag=q_tag, kv_tag=kv_tag, **kw)


# --------------------------------------------------------------------------
# pin checks (also reused against planted mistakes)
# --------------------------------------------------------------------------

def check_against_sdpa(mod):
    rng = np.random.default_rng(1)
    for g in (1, 2, 4, 8):
        for D in (8, 64):
            Hkv = 2 if g < 8 else 1
            Hq = g * Hkv
            lens = [1, 17, 70, 33][: 3 if g % 2 else 4]
            q, sk, sv = random_case(rng, len(lens), Hq, Hkv, D, lens)
            # storage is fp32, so the reference sees the same rounded values
            q = q.astype(np.float32).astype(np.float64)
            sk = [k.astype(np.float32).astype(np.float64) for k in sk]
            sv = [v.astype(np.float32).astype(np.float64) for v in sv]
            kc, vc, tables, L = paged_from_contiguous(sk, sv, 40, seed=g * 100 + D)
            scale = 1 / math.sqrt(D)
            got = run_oracle(mod, q, kc, vc, tables, L, scale)
            ref = sdpa_reference(q, sk, sv, scale)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def check_closed_forms(mod):
    rng = np.random.default_rng(2)
    D, Hkv, g = 16, 2, 4
    lens = [5, 16, 37]
    q, sk, sv = random_case(rng, 3, Hkv * g, Hkv, D, lens)
    # constant V -> output is that constant
    sv_c = [np.full_like(v, 0.625) for v in sv]
    kc, vc, t, L = paged_from_contiguous(sk, sv_c, 12, seed=3)
    got = run_oracle(mod, q, kc, vc, t, L, 0.25)
    np.testing.assert_allclose(got, 0.625, atol=1e-14)
    # zero query -> plain mean of V over the sequence
    kc, vc, t, L = paged_from_contiguous(sk, sv, 12, seed=4)
    got = run_oracle(mod, np.zeros_like(q), kc, vc, t, L, 0.25)
    for b in range(3):
        mean = sv[b].astype(np.float32).astype(np.float64).mean(axis=0)      # [Hkv, D]
        np.testing.assert_allclose(got[b], np.repeat(mean, g, axis=0), atol=1e-12)
    # one token -> that token's V
    q1, sk1, sv1 = random_case(rng, 2, Hkv * g, Hkv, D, [1, 1])
    kc, vc, t, L = paged_from_contiguous(sk1, sv1, 4, seed=5)
    got = run_oracle(mod, q1, kc, vc, t, L, 0.25)
    for b in range(2):
        np.testing.assert_allclose(got[b], np.repeat(sv1[b][0].astype(np.float32), g, axis=0), atol=1e-12)
    # one dominant key: q along that key with a large gap picks its V
    q2, sk2, sv2 = random_case(rng, 1, Hkv * g, Hkv, D, [29])
    sk2[0][:] = 0.0
    sk2[0][11] = 1.0
    q2[:] = 400.0                                  # score gap 400 * D * 0.25 for token 11
    kc, vc, t, L = paged_from_contiguous(sk2, sv2, 4, seed=6)
    got = run_oracle(mod, q2, kc, vc, t, L, 0.25)
    np.testing.assert_allclose(got[0], np.repeat(sv2[0][11].astype(np.float32), g, axis=0), atol=1e-12)
    # empty sequence -> zero row
    q3, sk3, sv3 = random_case(rng, 2, Hkv * g, Hkv, D, [0, 3])
    kc, vc, t, L = paged_from_contiguous(sk3, sv3, 4, seed=7)
    got = run_oracle(mod, q3, kc, vc, t, L, 0.25)
    assert np.all(got[0] == 0)


def check_invariances(mod):
    rng = np.random.default_rng(3)
    D, Hkv, g = 8, 2, 4
    lens = [19, 48, 3]
    q, sk, sv = random_case(rng, 3, Hkv * g, Hkv, D, lens)
    kc, vc, t, L = paged_from_contiguous(sk, sv, 20, seed=8)
    base = run_oracle(mod, q, kc, vc, t, L, 0.3)
    # physical permutation of blocks, tables remapped
    perm = np.random.default_rng(9).permutation(20)
    inv = np.argsort(perm)
    kp, vp = kc[perm], vc[perm]                     # new block j holds old block perm[j]
    tp = np.where(t >= 0, inv[np.maximum(t, 0)], -1).astype(np.int32)
    np.testing.assert_allclose(run_oracle(mod, q, kp, vp, tp, L, 0.3), base, atol=1e-13)
    # GQA == MHA with each K/V head duplicated g times (contiguous groups)
    skx = [np.repeat(k, g, axis=1) for k in sk]
    svx = [np.repeat(v, g, axis=1) for v in sv]
    kx, vx, tx, Lx = paged_from_contiguous(skx, svx, 20, seed=10)
    np.testing.assert_allclose(run_oracle(mod, q, kx, vx, tx, Lx, 0.3), base, atol=1e-13)
    # a shared 32-token prefix gives the same result as private copies
    pre_k = rng.standard_normal((32, Hkv, D))
    pre_v = rng.standard_normal((32, Hkv, D))
    sk2 = [np.concatenate([pre_k, k]) for k in sk]
    sv2 = [np.concatenate([pre_v, v]) for v in sv]
    ks, vs, ts, Ls = paged_from_contiguous(sk2, sv2, 30, seed=11, shared_prefix=32)
    kd, vd, td, Ld = paged_from_contiguous(sk2, sv2, 30, seed=12)
    assert (ts[:, :2] == ts[0, :2]).all()           # really shared
    np.testing.assert_allclose(run_oracle(mod, q, ks, vs, ts, Ls, 0.3),
                               run_oracle(mod, q, kd, vd, td, Ld, 0.3), atol=1e-13)


def check_window_against_masked_sdpa(mod):
    """Sliding window + sinks against float64 SDPA with an explicit mask built
    from the definition (the last W positions and the first S positions)."""
    rng = np.random.default_rng(11)
    D, Hkv, g = 16, 2, 2
    lens = [1, 7, 16, 17, 40, 70]
    q, sk, sv = random_case(rng, len(lens), Hkv * g, Hkv, D, lens)
    q = q.astype(np.float32).astype(np.float64)
    sk = [k.astype(np.float32).astype(np.float64) for k in sk]
    sv = [v.astype(np.float32).astype(np.float64) for v in sv]
    kc, vc, t, L = paged_from_contiguous(sk, sv, 20, seed=21)
    for W, S in [(1, 0), (5, 0), (16, 1), (17, 4), (33, 2), (500, 3), (3, 50)]:
        got = run_oracle(mod, q, kc, vc, t, L, 0.25, window=W, sinks=S)
        for b, Lb in enumerate(lens):
            pos = np.arange(Lb)
            keep = (pos >= Lb - W) | (pos < S)
            K = torch.from_numpy(sk[b]).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
            V = torch.from_numpy(sv[b]).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
            qq = torch.from_numpy(q[b])[:, None, :]
            mask = torch.from_numpy(keep)[None, None, :]
            ref = F.scaled_dot_product_attention(qq, K, V, attn_mask=mask, scale=0.25)[:, 0, :].numpy()
            np.testing.assert_allclose(got[b], ref, atol=1e-12)
    # window 1 without sinks: the newest token's V exactly
    got = run_oracle(mod, q, kc, vc, t, L, 0.25, window=1)
    for b, Lb in enumerate(lens):
        np.testing.assert_array_equal(got[b], np.repeat(sv[b][Lb - 1], g, axis=0))


PINS = [check_against_sdpa, check_closed_forms, check_invariances, check_window_against_masked_sdpa]


# --------------------------------------------------------------------------
# the pins themselves
# --------------------------------------------------------------------------

@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pins(pin):
    pin(oracle)


def test_storage_dtypes_decode_like_torch():
    """bf16 / f16 / fp8 caches: the oracle's values are torch's decoding."""
    rng = np.random.default_rng(4)
    D, Hkv, g = 16, 2, 2
    lens = [21, 40]
    q, sk, sv = random_case(rng, 2, Hkv * g, Hkv, D, lens)
    for tag, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        to_t = lambda a: torch.from_numpy(a).to(tdt)
        sk_t = [to_t(k) for k in sk]
        sv_t = [to_t(v) for v in sv]
        q_t = to_t(q)
        view = np.float16 if tag == "f16" else np.uint16
        bits = lambda t: (t.numpy() if tag == "f16" else t.view(torch.int16).numpy().view(np.uint16))
        kc, vc, t, L = paged_from_contiguous([bits(k) for k in sk_t], [bits(v) for v in sv_t], 8,
                                             seed=13, storage=view, fill=0)
        got = paged_decode_attention(bits(q_t), kc, vc, t, L, 0.25, q_tag=tag, kv_tag=tag)
        ref = sdpa_reference(q_t.double().numpy(), [k.double().numpy() for k in sk_t],
                             [v.double().numpy() for v in sv_t], 0.25)
        np.testing.assert_allclose(got, ref, atol=1e-12)
    # fp8 codes with one scale per (block, head): value = torch decode * scale
    codes_k = [rng.integers(0, 256, size=(L, Hkv, D)).astype(np.uint8) for L in lens]
    codes_v = [rng.integers(0, 256, size=(L, Hkv, D)).astype(np.uint8) for L in lens]
    for c in codes_k + codes_v:
        c[(c & 0x7F) == 0x7F] = 0x3C                # keep them finite
    kc, vc, t, L = paged_from_contiguous(codes_k, codes_v, 8, seed=14, storage=np.uint8, fill=0x7F)
    ks = rng.uniform(0.001, 0.01, size=(8, Hkv)).astype(np.float32)
    vs = rng.uniform(0.001, 0.01, size=(8, Hkv)).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16)
    got = paged_decode_attention(qb.view(torch.int16).numpy().view(np.uint16), kc, vc, t, L, 0.25,
                                 q_tag="bf16", kv_tag="fp8_e4m3", k_scales=ks, v_scales=vs)
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    # dequantised contiguous copies, block of each position found by brute force
    sk_d, sv_d = [], []
    for b in range(2):
        kd = np.zeros((lens[b], Hkv, D)); vd = np.zeros_like(kd)
        for pos in range(lens[b]):
            hits = [(blk, off) for blk in range(8) for off in range(BS)
                    if blk in t[b] and list(t[b]).index(blk) * BS + off == pos]
            (blk, off), = hits
            kd[pos] = dec(kc[blk, :, off, :]) * ks[blk][:, None]
            vd[pos] = dec(vc[blk, :, off, :]) * vs[blk][:, None]
        sk_d.append(kd); sv_d.append(vd)
    ref = sdpa_reference(qb.double().numpy(), sk_d, sv_d, 0.25)
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_page_of_matches_pool_bookkeeping_on_workloads():
    """For every workload, page_of() through the table finds each position at
    the slot the pool handed out when that token was added."""
    for w in WORKLOADS.values():
        if w.num_seqs * (w.len_range[1] if w.len_range else 100) > 2_000_000:
            w = scaled(w, num_seqs=2)
        lay = build_layout(w)
        for b in range(w.num_seqs):
            slots = lay.seq_slots[b]
            pos = np.arange(len(slots))
            blk, off = page_of(lay.block_tables[b], pos, BS)
            assert np.array_equal(blk * BS + off, slots)
            assert len(slots) == lay.context_lens[b]


def test_attended_positions_definition():
    from oracle import attended_positions
    assert list(attended_positions(10)) == list(range(10))
    assert list(attended_positions(10, window=3)) == [7, 8, 9]
    assert list(attended_positions(10, window=3, sinks=2)) == [0, 1, 7, 8, 9]
    assert list(attended_positions(4, window=3, sinks=2)) == [0, 1, 2, 3]
    assert list(attended_positions(0, window=3, sinks=2)) == []
    assert list(attended_positions(5, window=0, sinks=2)) == list(range(5))


def test_sequence_subset_selection():
    rng = np.random.default_rng(5)
    q, sk, sv = random_case(rng, 3, 8, 2, 16, [9, 20, 33])
    kc, vc, t, L = paged_from_contiguous(sk, sv, 10, seed=15)
    full = run_oracle(oracle, q, kc, vc, t, L, 0.25)
    part = run_oracle(oracle, q, kc, vc, t, L, 0.25, seqs=[2, 0], q_heads=[7, 1, 4])
    np.testing.assert_array_equal(part, full[[2, 0]][:, [7, 1, 4]])


def test_poisoned_slots_are_never_read():
    """Tails and unused blocks hold NaN; a finite output proves they are not read."""
    rng = np.random.default_rng(6)
    q, sk, sv = random_case(rng, 2, 4, 1, 8, [5, 31])
    kc, vc, t, L = paged_from_contiguous(sk, sv, 9, seed=16, fill=np.nan)
    assert np.isnan(kc).any()
    assert np.isfinite(run_oracle(oracle, q, kc, vc, t, L, 0.5)).all()


def test_tiny_workload_against_sdpa():
    """The tiny fp32 workload end to end: oracle append, then oracle attention,
    against SDPA on the per-position slots the pool recorded."""
    lay = build_layout(WORKLOADS["tiny_f32"])
    x = make_host_inputs(lay)
    kc = oracle.kv_append_bits(x["k_cache"][0].numpy(), x["k_new"][0].numpy(), lay.slot_mapping)
    vc = oracle.kv_append_bits(x["v_cache"][0].numpy(), x["v_new"][0].numpy(), lay.slot_mapping)
    q = x["q"][0].numpy()
    got = paged_decode_attention(q, kc, vc, lay.block_tables, lay.context_lens, 0.125, q_tag="f32", kv_tag="f32")
    sk = [np.stack([kc[s // BS, :, s % BS, :] for s in sl]).astype(np.float64) for sl in lay.seq_slots]
    sv = [np.stack([vc[s // BS, :, s % BS, :] for s in sl]).astype(np.float64) for sl in lay.seq_slots]
    ref = sdpa_reference(q.astype(np.float64), sk, sv, 0.125)
    np.testing.assert_allclose(got, ref, atol=1e-12)
    assert np.isfinite(got).all()


# --------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# --------------------------------------------------------------------------

MUTANTS = {
    "head_map_modulo": ("h = col[kv_for[c]]", "h = col[kv_for[c]] if False else (q_heads[c] % Hkv) % len(kv_needed)"),
    "scale_dropped": ("s = scale * (K[:, h, :] @ qv[r, c])", "s = (K[:, h, :] @ qv[r, c])"),
    "length_off_by_one": ("L = int(context_lens[b])", "L = max(int(context_lens[b]) - 1, 0)"),
    "offset_uses_block_index": ("return np.asarray(table_row)[logical_page], offset",
                                "return np.asarray(table_row)[logical_page], logical_page % int(block_size)"),
    "k_v_swapped": ("out[r, c] = (w @ V[:, h, :]) / w.sum()", "out[r, c] = (w @ K[:, h, :]) / w.sum()"),
    "normalise_by_length": ("out[r, c] = (w @ V[:, h, :]) / w.sum()", "out[r, c] = (w @ V[:, h, :]) / len(w)"),
    "exponent_sign": ("w = np.exp(s - s.max())", "w = np.exp(s.max() - s)"),
    "fp8_scale_ignored": ("vals = vals * s[blk[:, None], kv_heads[None, :]][:, :, None]", "vals = vals"),
    "window_off_by_one": ("recent = np.arange(max(0, L - int(window)), L)",
                          "recent = np.arange(max(0, L - int(window) + 1), L)"),
    "sinks_ignored": ("first = np.arange(min(int(sinks), L))", "first = np.arange(0)"),
    "channel_factors_dropped": ("vals = vals * c[kv_heads][None, :, :]", "vals = vals"),
    "channel_factors_transposed": ("vals = vals * c[kv_heads][None, :, :]",
                                   "vals = vals * c[kv_heads][None, :, ::-1]"),
    "v_read_in_k_format": ("V = gather_sequence(v_cache, block_tables[b], L, v_tag,",
                           "V = gather_sequence(v_cache, block_tables[b], L, kv_tag,"),
    "side_sinks_ignored": ("        if side and len(first):", "        if False:"),
    "side_sink_offset": ("[kv_needed][:, first, :].transpose(1, 0, 2)   # [n, h, D]",
                         "[kv_needed][:, first[::-1], :].transpose(1, 0, 2)   # [n, h, D]"),
    "token_scale_offset_ignored": ("vals = vals * s[blk[:, None], kv_heads[None, :], off[:, None]][:, :, None]",
                                   "vals = vals * s[blk[:, None], kv_heads[None, :], 0 * off[:, None]][:, :, None]"),
    "token_scale_offset_reversed": ("vals = vals * s[blk[:, None], kv_heads[None, :], off[:, None]][:, :, None]",
                                    "vals = vals * s[blk[:, None], kv_heads[None, :], (block_size - 1 - off)[:, None]][:, :, None]"),
    "query_head_index": ("qv = stored_to_f64(np.asarray(q)[seqs][:, q_heads], q_tag)",
                         "qv = stored_to_f64(np.asarray(q)[seqs][:, q_heads][:, ::-1], q_tag)"),
}


def _mutant_module(name):
    import inspect
    import oracle.paged_attention as pa
    src = inspect.getsource(pa)
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__dict__["__name__"] = mod.__name__
    src = src.replace("from .values import stored_to_f64", "from oracle.values import stored_to_f64")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _fp8_pin(mod):
    """Same as the fp8 part of test_storage_dtypes_decode_like_torch, as a pin."""
    rng = np.random.default_rng(8)
    lens = [20]
    codes_k = [rng.integers(0, 0x70, size=(20, 1, 8)).astype(np.uint8)]
    codes_v = [rng.integers(0, 0x70, size=(20, 1, 8)).astype(np.uint8)]
    kc, vc, t, L = paged_from_contiguous(codes_k, codes_v, 3, seed=17, storage=np.uint8, fill=0x7F)
    ks = np.full((3, 1), 0.5, np.float32)
    vs = np.full((3, 1), 0.25, np.float32)
    q = rng.standard_normal((1, 2, 8)).astype(np.float32)
    got = mod.paged_decode_attention(q, kc, vc, t, L, 0.3, q_tag="f32", kv_tag="fp8_e4m3", k_scales=ks, v_scales=vs)
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    ref = sdpa_reference(q.astype(np.float64), [dec(codes_k[0]) * 0.5], [dec(codes_v[0]) * 0.25], 0.3)
    np.testing.assert_allclose(got, ref, atol=1e-12)


def _mixed_pin(mod):
    """fp8 K with per-channel factors and int8 V: the dense reference uses
    K = decode(code) * block scale * channel factor and V = code * block
    scale, built position by position (torch's fp8 decode, numpy's int8)."""
    rng = np.random.default_rng(9)
    lens = [19, 35]
    Hkv, D = 2, 8
    codes_k = [rng.integers(0, 0x70, size=(L, Hkv, D)).astype(np.uint8) for L in lens]
    codes_v = [rng.integers(-127, 128, size=(L, Hkv, D)).astype(np.int8) for L in lens]
    kc, _, t, Ls = paged_from_contiguous(codes_k, codes_k, 6, seed=18, storage=np.uint8, fill=0x7F)
    vc, _, t2, _ = paged_from_contiguous(codes_v, codes_v, 6, seed=18, storage=np.int8, fill=0)
    assert np.array_equal(t, t2)
    ks = rng.uniform(0.01, 0.1, size=(6, Hkv)).astype(np.float32)
    vs = rng.uniform(0.01, 0.1, size=(6, Hkv)).astype(np.float32)
    cs = rng.uniform(0.5, 4.0, size=(Hkv, D)).astype(np.float32)
    q = rng.standard_normal((2, 4, D)).astype(np.float32)
    got = mod.paged_decode_attention(q, kc, vc, t, Ls, 0.4, q_tag="f32", kv_tag="fp8_e4m3",
                                     v_tag="int8", k_scales=ks, v_scales=vs, k_channel_scales=cs)
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    sk_d, sv_d = [], []
    for b, L in enumerate(lens):
        kd = np.zeros((L, Hkv, D)); vd = np.zeros_like(kd)
        for pos in range(L):
            blk = t[b][pos // BS]
            kd[pos] = dec(codes_k[b][pos]) * ks[blk][:, None] * cs
            vd[pos] = codes_v[b][pos].astype(np.float64) * vs[blk][:, None]
        sk_d.append(kd); sv_d.append(vd)
    ref = sdpa_reference(q.astype(np.float64), sk_d, sv_d, 0.4)
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_mixed_precision_pin():
    _mixed_pin(oracle)


def _token_scale_pin(mod):
    """fp8 K and int8 V with one scale per (slot, head): the dense reference
    multiplies each token's row by the scale of its own slot, built
    position by position."""
    rng = np.random.default_rng(12)
    lens = [21, 40]
    Hkv, D = 2, 8
    codes_k = [rng.integers(0, 0x70, size=(L, Hkv, D)).astype(np.uint8) for L in lens]
    codes_v = [rng.integers(-127, 128, size=(L, Hkv, D)).astype(np.int8) for L in lens]
    kc, _, t, Ls = paged_from_contiguous(codes_k, codes_k, 7, seed=22, storage=np.uint8, fill=0x7F)
    vc, _, t2, _ = paged_from_contiguous(codes_v, codes_v, 7, seed=22, storage=np.int8, fill=0)
    assert np.array_equal(t, t2)
    ks = rng.uniform(0.001, 0.1, size=(7, Hkv, BS)).astype(np.float32)
    vs = rng.uniform(0.001, 0.1, size=(7, Hkv, BS)).astype(np.float32)
    q = rng.standard_normal((2, 4, D)).astype(np.float32)
    got = mod.paged_decode_attention(q, kc, vc, t, Ls, 0.4, q_tag="f32", kv_tag="fp8_e4m3",
                                     v_tag="int8", k_scales=ks, v_scales=vs)
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    sk_d, sv_d = [], []
    for b, L in enumerate(lens):
        kd = np.zeros((L, Hkv, D)); vd = np.zeros_like(kd)
        for pos in range(L):
            blk, off = t[b][pos // BS], pos % BS
            kd[pos] = dec(codes_k[b][pos]) * ks[blk, :, off][:, None]
            vd[pos] = codes_v[b][pos].astype(np.float64) * vs[blk, :, off][:, None]
        sk_d.append(kd); sv_d.append(vd)
    ref = sdpa_reference(q.astype(np.float64), sk_d, sv_d, 0.4)
    np.testing.assert_allclose(got, ref, atol=1e-12)


def _k16_v8_pin(mod):
    """K kept in f16 (as stored, no scale) with V in fp8 (block scales) or
    int8 (per-token scales): the dense reference reads K as f16 values and
    V as code times scale, position by position."""
    rng = np.random.default_rng(13)
    lens = [17, 33, 5]
    Hkv, D = 1, 8
    k16 = [rng.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
    codes_f8 = [rng.integers(0, 0x70, size=(L, Hkv, D)).astype(np.uint8) for L in lens]
    codes_i8 = [rng.integers(-127, 128, size=(L, Hkv, D)).astype(np.int8) for L in lens]
    kc, _, t, Ls = paged_from_contiguous(k16, k16, 6, seed=23, storage=np.float16, fill=np.nan)
    v8, _, t2, _ = paged_from_contiguous(codes_f8, codes_f8, 6, seed=23, storage=np.uint8, fill=0x7F)
    vi, _, t3, _ = paged_from_contiguous(codes_i8, codes_i8, 6, seed=23, storage=np.int8, fill=0)
    assert np.array_equal(t, t2) and np.array_equal(t, t3)
    vs_blk = rng.uniform(0.01, 0.1, size=(6, Hkv)).astype(np.float32)
    vs_tok = rng.uniform(0.01, 0.1, size=(6, Hkv, BS)).astype(np.float32)
    q = rng.standard_normal((3, 4, D)).astype(np.float16)
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    for vcache, vtag, vs in ((v8, "fp8_e4m3", vs_blk), (vi, "int8", vs_tok)):
        got = mod.paged_decode_attention(q, kc, vcache, t, Ls, 0.35, q_tag="f16", kv_tag="f16",
                                         v_tag=vtag, v_scales=vs)
        sk_d, sv_d = [], []
        for b, L in enumerate(lens):
            kd = np.zeros((L, Hkv, D)); vd = np.zeros_like(kd)
            for pos in range(L):
                blk, off = t[b][pos // BS], pos % BS
                kd[pos] = k16[b][pos].astype(np.float64)
                if vtag == "fp8_e4m3":
                    vd[pos] = dec(codes_f8[b][pos]) * vs[blk][:, None]
                else:
                    vd[pos] = codes_i8[b][pos].astype(np.float64) * vs[blk, :, off][:, None]
            sk_d.append(kd); sv_d.append(vd)
        ref = sdpa_reference(q.astype(np.float64), sk_d, sv_d, 0.35)
        np.testing.assert_allclose(got, ref, atol=1e-12)


def test_per_token_scale_pin():
    _token_scale_pin(oracle)


def test_k16_with_v8_pin():
    _k16_v8_pin(oracle)


def _side_sink_pin(mod):
    """int8 cache with the first S positions of each sequence in f16 side
    tiles: the dense reference takes positions < S from the tile, as stored,
    and the rest from the int8 cache, with and without a window."""
    rng = np.random.default_rng(10)
    lens = [3, 16, 40]
    Hkv, D, S = 2, 8, 5
    codes_k = [rng.integers(-127, 128, size=(L, Hkv, D)).astype(np.int8) for L in lens]
    codes_v = [rng.integers(-127, 128, size=(L, Hkv, D)).astype(np.int8) for L in lens]
    kc, vc, t, Ls = paged_from_contiguous(codes_k, codes_v, 8, seed=19, storage=np.int8, fill=-128)
    ks = rng.uniform(0.01, 0.1, size=(8, Hkv)).astype(np.float32)
    vs = rng.uniform(0.01, 0.1, size=(8, Hkv)).astype(np.float32)
    tiles = (rng.standard_normal((2, 5, Hkv, BS, D)) * 8).astype(np.float16)     # K, V side tiles
    sink_blocks = np.array([4, 0, 2])
    q = rng.standard_normal((3, 4, D)).astype(np.float16)
    for window in (0, 12):
        got = mod.paged_decode_attention(q, kc, vc, t, Ls, 0.3, q_tag="f16", kv_tag="int8",
                                         k_scales=ks, v_scales=vs, window=window, sinks=S,
                                         sink_k=tiles[0], sink_v=tiles[1], sink_blocks=sink_blocks)
        sk_d, sv_d = [], []
        for b, L in enumerate(lens):
            keep = [p for p in range(L) if window == 0 or p >= L - window or p < S]
            kd = np.zeros((len(keep), Hkv, D)); vd = np.zeros_like(kd)
            for r, pos in enumerate(keep):
                blk = t[b][pos // BS]
                if pos < S:
                    kd[r] = tiles[0][sink_blocks[b], :, pos, :].astype(np.float64)
                    vd[r] = tiles[1][sink_blocks[b], :, pos, :].astype(np.float64)
                else:
                    kd[r] = codes_k[b][pos].astype(np.float64) * ks[blk][:, None]
                    vd[r] = codes_v[b][pos].astype(np.float64) * vs[blk][:, None]
            sk_d.append(kd); sv_d.append(vd)
        ref = sdpa_reference(q.astype(np.float64), sk_d, sv_d, 0.3)
        np.testing.assert_allclose(got, ref, atol=1e-12)


def test_full_precision_sink_pin():
    _side_sink_pin(oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant_module(name)
    caught = []
    for pin in PINS + [_fp8_pin, _mixed_pin, _side_sink_pin, _token_scale_pin, _k16_v8_pin]:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
