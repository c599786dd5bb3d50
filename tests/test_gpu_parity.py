"""HIP path against the float64 oracle, element by element (needs a GPU).

Tolerances (max-abs against the oracle run on the same stored values):
fp32 1e-5, fp16/bf16 1e-2, 8-bit caches (fp8, int8, mixed) 5e-2; every
append (plain or quantising) bit-exact.  The one final rounding of the
result to the output type (half an ulp at the oracle's value) is not charged
against the tolerance only where half an ulp of the output type at the
oracle's value is itself above the tolerance (bf16 outputs of 4 or more,
from the full-precision sink tiles); everywhere else the raw max-abs error
is what is asserted (gpu_common.parity_err).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_56_amd as pkv
from workloads import (WORKLOADS, DecodeWorkload, build_layout, make_host_inputs, make_device_inputs, scaled,
                       share_prefixes)
from gpu_common import (TOL, say, host_storage, run_step, oracle_rows, oracle_append, oracle_attend,
                        host_layer, out_f64, max_err, parity_err)

pytestmark = pytest.mark.gpu

DEV = "cuda"
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _to_dev(x):
    return {k: v.to(DEV) for k, v in x.items()}


def _out(spec, layers=None):
    return torch.empty((spec.num_seqs, spec.num_q_heads, spec.head_dim),
                       dtype=TORCH_DT[spec.out_dtype], device=DEV)


# --------------------------------------------------------------------------
# kv_append
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_kv_append_bit_exact(dt):
    say(f"[kv_append] dtype={dt}")
    spec = DecodeWorkload(name=f"append_{dt}", seed=77, num_layers=1, num_seqs=9, num_q_heads=8,
                          num_kv_heads=4, head_dim=128, kv_dtype=dt, q_dtype=dt, out_dtype=dt,
                          context_lens=(1, 16, 17, 32, 33, 100, 255, 256, 257), num_blocks=80)
    lay = build_layout(spec)
    x = make_host_inputs(lay)
    slots = lay.slot_mapping.copy()
    slots[3] = -1                                    # skipped token
    xs = _to_dev(x)
    sm = torch.from_numpy(slots).to(DEV)
    pkv.kv_append(xs["k_new"][0], xs["v_new"][0], sm, xs["k_cache"][0], xs["v_cache"][0])
    torch.cuda.synchronize()
    for name, new in (("k_cache", "k_new"), ("v_cache", "v_new")):
        ref = oracle.kv_append_bits(host_storage(x[name][0]), host_storage(x[new][0]), slots)
        got = host_storage(xs[name][0])
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), name


@pytest.mark.parametrize("src", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("first_write", [False, True])
def test_kv_append_fp8_bit_exact(src, first_write):
    """Codes and scales equal the oracle's bit for bit, including several
    tokens of one call landing in one fresh block (first-write ordering)."""
    say(f"[kv_append_fp8] src={src} first_write={first_write}")
    rng = np.random.default_rng(5)
    NB, H, D, T = 12, 4, 128, 21
    codes = rng.integers(0, 0x7E, size=(NB, H, 16, D)).astype(np.uint8)
    scales = rng.uniform(0.002, 0.05, size=(NB, H)).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((T, H, D)).astype(np.float32) * 2).to(TORCH_DT[src])
    x[3] *= 40                                           # exceeds 448 * scale somewhere
    slots = np.array([0, 1, 2, 3, 4, 5, 16, 33, -1, 48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 190,
                      NB * 16 + 3], dtype=np.int64)
    xs = host_storage(x)
    xf = oracle.stored_to_f64(xs, src).astype(np.float32)
    ref_c, ref_s = oracle.kv_append_fp8(codes, scales, xf, slots, first_write=first_write)
    dc = torch.from_numpy(codes).to(DEV)
    dv = torch.from_numpy(codes).to(DEV)
    ks = torch.from_numpy(scales).to(DEV)
    vs = torch.from_numpy(scales).to(DEV)
    xd = x.to(DEV)
    pkv.kv_append_fp8(xd, xd, torch.from_numpy(slots).to(DEV), dc, dv, ks, vs, first_write=first_write)
    torch.cuda.synchronize()
    for c_, s_ in ((dc, ks), (dv, vs)):
        assert np.array_equal(c_.cpu().numpy(), ref_c)
        assert np.array_equal(s_.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def test_fp8_quantise_ties_saturation_and_subnormals():
    """Scale 1: the codes are the hardware's RNE e4m3 of the clamped values --
    every tie between neighbouring codes and both fp32 neighbours of it,
    the subnormal range, zeros, and values past 448 (including infinity)."""
    say("[kv_append_fp8] rounding edge cases")
    vals = np.sort(oracle.decode_e4m3fn(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    edge = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
                           np.float32([0.0, -0.0, 447.9, 448.0, 449.0, 464.0, 465.0, 1e6, np.inf, 2.0**-10,
                                       2.0**-11, 3 * 2.0**-11, 1e-30])]).astype(np.float32)
    edge = np.concatenate([edge, -edge])
    D, H = 128, 1
    T = -(-edge.size // D)
    x = np.zeros((T * D,), np.float32)
    x[: edge.size] = edge
    x = x.reshape(T, H, D)
    NB = -(-T // 16)
    slots = np.arange(T, dtype=np.int64)
    codes = np.zeros((NB, H, 16, D), np.uint8)
    ones = np.ones((NB, H), np.float32)
    ref_c, _ = oracle.kv_append_fp8(codes, ones, x, slots, first_write=False)
    dc = torch.zeros((NB, H, 16, D), dtype=torch.uint8, device=DEV)
    dv = torch.zeros_like(dc)
    s1 = torch.ones((NB, H), device=DEV)
    s2 = torch.ones((NB, H), device=DEV)
    xd = torch.from_numpy(x).to(DEV)
    pkv.kv_append_fp8(xd, xd, torch.from_numpy(slots).to(DEV), dc, dv, s1, s2)
    torch.cuda.synchronize()
    got = dc.cpu().numpy()
    bad = np.argwhere(got != ref_c)
    assert bad.size == 0, [(tuple(i), int(got[tuple(i)]), int(ref_c[tuple(i)])) for i in bad[:8]]


@pytest.mark.parametrize("code", ["int8", "fp8_e4m3"])
@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("first_write", [False, True])
@pytest.mark.parametrize("chan", [False, True])
def test_kv_append_quant_bit_exact(code, src, first_write, chan):
    """One cache at a time, with or without per-channel factors: codes and
    scales equal the oracle's bit for bit."""
    say(f"[kv_append_quant] code={code} src={src} first_write={first_write} chan={chan}")
    rng = np.random.default_rng(11)
    NB, H, D, T = 12, 4, 128, 21
    npdt = np.uint8 if code == "fp8_e4m3" else np.int8
    codes = rng.integers(0, 0x7E, size=(NB, H, 16, D)).astype(npdt)
    scales = rng.uniform(0.002, 0.05, size=(NB, H)).astype(np.float32)
    cs = None
    if chan:
        cs = rng.uniform(0.25, 20.0, size=(H, D)).astype(np.float32)
        cs[:, ::7] = 16.0
    x = torch.from_numpy(rng.standard_normal((T, H, D)).astype(np.float32) * 2).to(TORCH_DT[src])
    x[3] *= 40
    slots = np.array([0, 1, 2, 3, 4, 5, 16, 33, -1, 48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 190,
                      NB * 16 + 3], dtype=np.int64)
    xf = oracle.stored_to_f64(host_storage(x), src).astype(np.float32)
    ref_c, ref_s = oracle.kv_append_quant(codes, scales, xf, slots, code=code, first_write=first_write,
                                          channel_scales=cs)
    dc = torch.from_numpy(codes).to(DEV)
    ds = torch.from_numpy(scales).to(DEV)
    dcs = None if cs is None else torch.from_numpy(cs).to(DEV)
    pkv.kv_append_quant(x.to(DEV), torch.from_numpy(slots).to(DEV), dc, ds, channel_scales=dcs,
                        first_write=first_write)
    torch.cuda.synchronize()
    assert np.array_equal(dc.cpu().numpy(), ref_c)
    assert np.array_equal(ds.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


@pytest.mark.parametrize("code", ["int8", "fp8_e4m3"])
@pytest.mark.parametrize("src", ["f16", "bf16"])
@pytest.mark.parametrize("chan", [False, True])
def test_kv_append_quant_per_token_bit_exact(code, src, chan):
    """One scale per (slot, head): every written token sets its own scales
    from its row; codes and scales equal the oracle's bit for bit, and no
    other slot's scale changes."""
    say(f"[kv_append_quant per token] code={code} src={src} chan={chan}")
    rng = np.random.default_rng(12)
    NB, H, D, T = 10, 3, 128, 19
    npdt = np.uint8 if code == "fp8_e4m3" else np.int8
    codes = rng.integers(0, 0x7E, size=(NB, H, 16, D)).astype(npdt)
    scales = rng.uniform(0.002, 0.05, size=(NB, H, 16)).astype(np.float32)
    cs = None
    if chan:
        cs = rng.uniform(0.25, 20.0, size=(H, D)).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((T, H, D)).astype(np.float32) * 2).to(TORCH_DT[src])
    x[3] *= 40
    x[5] = 0                                       # a zero row: scale 1
    slots = np.array([0, 1, 2, 3, 4, 5, 16, 33, -1, 48, 49, 50, 51, 52, 53, 54, 55, 159,
                      NB * 16 + 3], dtype=np.int64)
    xf = oracle.stored_to_f64(host_storage(x), src).astype(np.float32)
    ref_c, ref_s = oracle.kv_append_quant(codes, scales, xf, slots, code=code, first_write=False,
                                          channel_scales=cs, granularity="token")
    dc = torch.from_numpy(codes).to(DEV)
    ds = torch.from_numpy(scales).to(DEV)
    dcs = None if cs is None else torch.from_numpy(cs).to(DEV)
    pkv.kv_append_quant(x.to(DEV), torch.from_numpy(slots).to(DEV), dc, ds, channel_scales=dcs)
    torch.cuda.synchronize()
    assert np.array_equal(dc.cpu().numpy(), ref_c)
    assert np.array_equal(ds.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def test_kv_append_k_alone():
    """pkv_kv_append with no V: the K rows are bit-copied, nothing else moves."""
    say("[kv_append] K alone")
    rng = np.random.default_rng(13)
    kc = torch.from_numpy(rng.standard_normal((6, 2, 16, 128)).astype(np.float32)).to(torch.bfloat16)
    new = torch.from_numpy(rng.standard_normal((4, 2, 128)).astype(np.float32)).to(torch.bfloat16)
    slots = np.array([3, 17, -1, 95], dtype=np.int64)
    ref = oracle.kv_append_bits(host_storage(kc), host_storage(new), slots)
    dk = kc.to(DEV)
    pkv.kv_append(new.to(DEV), None, torch.from_numpy(slots).to(DEV), dk, None)
    torch.cuda.synchronize()
    assert np.array_equal(host_storage(dk), ref)


def test_int8_quantise_ties_saturation_and_nan():
    """Scale 1: every half-integer tie in range, both fp32 neighbours of it,
    +-127.5 and beyond, infinities and NaN."""
    say("[kv_append_quant] int8 rounding edge cases")
    half = np.arange(-127, 127, dtype=np.float32) + np.float32(0.5)
    edge = np.concatenate([half, np.nextafter(half, np.float32(-np.inf)), np.nextafter(half, np.float32(np.inf)),
                           np.float32([0.0, -0.0, 126.9, 127.0, 127.49, 127.5, 128.0, 1e6, np.inf, -np.inf,
                                       np.nan, 1e-30, -1e-30])]).astype(np.float32)
    D, H = 128, 1
    T = -(-edge.size // D)
    x = np.zeros((T * D,), np.float32)
    x[: edge.size] = edge
    x = x.reshape(T, H, D)
    NB = -(-T // 16)
    slots = np.arange(T, dtype=np.int64)
    codes = np.zeros((NB, H, 16, D), np.int8)
    ones = np.ones((NB, H), np.float32)
    ref_c, _ = oracle.kv_append_int8(codes, ones, x, slots, first_write=False)
    dc = torch.zeros((NB, H, 16, D), dtype=torch.int8, device=DEV)
    pkv.kv_append_quant(torch.from_numpy(x).to(DEV), torch.from_numpy(slots).to(DEV), dc,
                        torch.ones((NB, H), device=DEV))
    torch.cuda.synchronize()
    got = dc.cpu().numpy()
    bad = np.argwhere(got != ref_c)
    assert bad.size == 0, [(tuple(i), int(got[tuple(i)]), int(ref_c[tuple(i)])) for i in bad[:8]]


def test_int8_all_codes_decode_through_attention():
    """With one token, out = V * scale: every int8 code (scale 1, and a
    power-of-two scale) comes out exactly, under fp8 and int8 K."""
    say("[int8] 256 codes through a length-1 attention")
    D = 128
    codes = np.arange(-128, 128, dtype=np.int16).astype(np.int8).reshape(2, D)
    vc = np.zeros((4, 1, 16, D), np.int8)
    vc[1, 0, 0] = codes[0]
    vc[3, 0, 0] = codes[1]
    tables = np.array([[1], [3]], np.int32)
    lens = np.array([1, 1], np.int32)
    q = torch.randn((2, 1, D), device=DEV).to(torch.bfloat16)
    for kdt, kfill in ((torch.uint8, 0x38), (torch.int8, 5)):
        kc = torch.full((4, 1, 16, D), kfill, dtype=kdt, device=DEV)
        for vscale in (1.0, 0.25):
            out = torch.empty((2, 1, D), device=DEV, dtype=torch.bfloat16)
            vs = torch.full((4, 1), vscale, device=DEV)
            pkv.paged_decode_attn(q, kc, torch.from_numpy(vc).to(DEV), torch.from_numpy(tables).to(DEV),
                                  torch.from_numpy(lens).to(DEV), 0.1, out,
                                  k_scales=torch.ones((4, 1), device=DEV), v_scales=vs)
            got = out.float().cpu().numpy()[:, 0, :].astype(np.float64)
            assert np.array_equal(got, codes.astype(np.float64) * vscale), (kdt, vscale)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16", "fp8_e4m3", "int8"])
def test_copy_blocks_bit_exact(dt):
    say(f"[copy_blocks] dtype={dt}")
    rng = np.random.default_rng(9)
    NB, H, D = 40, 4, 128
    nbytes = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1, "int8": 1}[dt]
    raw = rng.integers(0, 256, size=(2, NB, H, 16, D * nbytes), dtype=np.uint8)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8,
           "int8": torch.int8}[dt]
    kc = torch.from_numpy(raw[0].copy()).view(tdt).to(DEV)
    vc = torch.from_numpy(raw[1].copy()).view(tdt).to(DEV)
    src = np.array([3, 7, 11, 0, 39, 5, 2], np.int32)
    dst = np.array([20, 21, 22, 23, 24, 99, 2], np.int32)     # 99 outside the pool, 2 -> 2 no-op
    ks = vs = None
    sc = rng.uniform(size=(2, NB, H)).astype(np.float32)
    if dt in ("fp8_e4m3", "int8"):
        ks, vs = torch.from_numpy(sc[0].copy()).to(DEV), torch.from_numpy(sc[1].copy()).to(DEV)
    pkv.copy_blocks(kc, vc, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV), ks, vs)
    torch.cuda.synchronize()
    for t, c_ in enumerate((kc, vc)):
        exp = raw[t].copy()
        for s_, d_ in zip(src, dst):
            if d_ < NB and s_ != d_:
                exp[d_] = raw[t][s_]
        got = c_.cpu().contiguous().view(torch.uint8).numpy().reshape(exp.shape)
        assert np.array_equal(got, exp)
        if ks is not None:
            e2 = sc[t].copy()
            for s_, d_ in zip(src, dst):
                if d_ < NB and s_ != d_:
                    e2[d_] = sc[t][s_]
            assert np.array_equal((ks, vs)[t].cpu().numpy(), e2)


def test_fork_copy_on_write_end_to_end():
    """A parent with a partial last block is forked three times; parent and
    children then append different tokens.  The native manager and the
    oracle's reference manager (oracle.block_manager) are driven with the
    same calls and must hand out the same slots and copies; the device runs
    the copies and appends, the host applies the same copies and the
    oracle's append to its own copy of the caches.  The caches must then be
    bit-identical, and attention for every sequence must equal the oracle's
    attention over the reference manager's tables."""
    from oracle.block_manager import ReferenceBlockManager

    say("[cow] fork + copy-on-write + append + attention")
    rng = np.random.default_rng(12)
    NB, H, G, D = 24, 2, 4, 64
    order = rng.permutation(NB).tolist()
    bm = pkv.BlockManager(NB, free_order=order)
    ref_bm = ReferenceBlockManager(NB, free_order=order)
    kc = torch.full((NB, H, 16, D), float("nan"), dtype=torch.float16, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    hk, hv = host_storage(kc).copy(), host_storage(vc).copy()
    bm.add_sequence(0)
    ref_bm.add_sequence(0)
    gen = torch.Generator().manual_seed(12)

    def step(seqs):
        slots, copies = bm.append_slots(seqs)
        rslots, rcopies = ref_bm.append_slots(seqs)
        assert slots == rslots and copies == rcopies
        if copies:
            cs = torch.tensor([c[0] for c in copies], dtype=torch.int32, device=DEV)
            cd = torch.tensor([c[1] for c in copies], dtype=torch.int32, device=DEV)
            pkv.copy_blocks(kc, vc, cs, cd)
            for src, dst in rcopies:
                hk[dst], hv[dst] = hk[src], hv[src]
        kn = torch.randn((len(seqs), H, D), generator=gen).to(torch.float16)
        vn = torch.randn((len(seqs), H, D), generator=gen).to(torch.float16)
        pkv.kv_append(kn.to(DEV), vn.to(DEV), torch.tensor(slots, dtype=torch.int64, device=DEV), kc, vc)
        sl = np.array(rslots, dtype=np.int64)
        hk[...] = oracle.kv_append_bits(hk, kn.numpy(), sl)
        hv[...] = oracle.kv_append_bits(hv, vn.numpy(), sl)
        return copies

    for _ in range(20):
        step([0])
    for c in (1, 2, 3):
        bm.fork(0, c)
        ref_bm.fork(0, c)
    ncopies = 0
    for r in range(17):
        ncopies += len(step([3, 0, 1, 2] if r % 2 else [1, 2, 3, 0]))
    # the partial block was shared four ways: the first three writers copy it,
    # the last one is then its only holder and writes in place
    assert ncopies == 3
    seqs = [0, 1, 2, 3]
    tables, lens = bm.block_tables(seqs, 4)
    ref_tables = np.full((4, 4), -1, dtype=np.int32)
    for i, s_ in enumerate(seqs):
        ref_tables[i, :len(ref_bm.tables[s_])] = ref_bm.tables[s_]
    ref_lens = np.array([ref_bm.lens[s_] for s_ in seqs], dtype=np.int32)
    assert np.array_equal(tables.numpy(), ref_tables) and np.array_equal(lens.numpy(), ref_lens)
    torch.cuda.synchronize()
    assert np.array_equal(host_storage(kc).view(np.uint16), hk.view(np.uint16))
    assert np.array_equal(host_storage(vc).view(np.uint16), hv.view(np.uint16))
    q = torch.randn((4, H * G, D), generator=gen).to(torch.float16)
    out = torch.empty((4, H * G, D), dtype=torch.float16, device=DEV)
    pkv.paged_decode_attn(q.to(DEV), kc, vc, tables.to(DEV), lens.to(DEV), 0.125, out)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(q.numpy(), hk, hv, ref_tables, ref_lens, 0.125,
                                        q_tag="f16", kv_tag="f16")
    err = parity_err(out_f64(out), ref, "f16", TOL["f16"])
    say(f"    max|err| = {err:.3e} (tol {TOL['f16']})")
    assert err <= TOL["f16"]
    bm.close()


def test_kv_append_skips_out_of_pool_slots():
    say("[kv_append] out-of-pool slot")
    kc = torch.zeros((2, 1, 16, 64), dtype=torch.float16, device=DEV)
    vc = torch.zeros_like(kc)
    new = torch.ones((3, 1, 64), dtype=torch.float16, device=DEV)
    sm = torch.tensor([5, 2 * 16, 31], dtype=torch.int64, device=DEV)
    pkv.kv_append(new, new, sm, kc, vc)
    torch.cuda.synchronize()
    flat = kc.view(32, 64).cpu()
    assert (flat[5] == 1).all() and (flat[31] == 1).all()
    assert flat.sum().item() == 2 * 64


# --------------------------------------------------------------------------
# decode attention, oracle-sized cases
# --------------------------------------------------------------------------

def _ragged(name, kv, q, out, D, G, lens, seed, hkv=2, append=False, v=None, outliers=0, fp_sinks=0,
            ktok=False, vtok=False):
    return DecodeWorkload(name=name, seed=seed, num_layers=1, num_seqs=len(lens), num_q_heads=hkv * G,
                          num_kv_heads=hkv, head_dim=D, kv_dtype=kv, q_dtype=q, out_dtype=out,
                          context_lens=tuple(lens), append=append, v_dtype=v, k_outliers=outliers,
                          fp_sinks=fp_sinks, k_scale_tok=ktok, v_scale_tok=vtok)


RAGGED = [1, 15, 16, 17, 31, 33, 100, 257, 0, 64, 511]
APPEND_STEPS = [129, 144, 177, 192, 113, 128, 33, 48, 49, 65]
SMALL = {
    "tiny_f32": WORKLOADS["tiny_f32"],
    "llama3_8b_bf16_small": scaled(WORKLOADS["llama3_8b_bf16"], num_seqs=4, len_range=(512, 2100)),
    "llama70b_f16_small": scaled(WORKLOADS["llama70b_f16_80l"], num_layers=2, num_seqs=3),
    "mha13b_prefix_small": scaled(WORKLOADS["mha13b_prefix_f16"], num_seqs=6),
    "long_fp8_small": scaled(WORKLOADS["long_fp8"], num_seqs=2, len_range=(8192, 8192)),
    "llama70b_fp8_small": scaled(WORKLOADS["llama70b_fp8_80l"], num_layers=2, num_seqs=3),
    "ragged_f16_g8_d128": _ragged("r1", "f16", "f16", "f16", 128, 8, RAGGED, 1),
    "ragged_bf16_g4_d64": _ragged("r2", "bf16", "bf16", "bf16", 64, 4, RAGGED, 2),
    "ragged_f32_g8_d128": _ragged("r3", "f32", "f32", "f32", 128, 8, RAGGED, 3),
    "ragged_f16_g2_d64": _ragged("r4", "f16", "f16", "f16", 64, 2, RAGGED, 4),
    "ragged_f32_g1_d64": _ragged("r5", "f32", "f32", "f32", 64, 1, RAGGED, 5),
    "ragged_fp8_g8_d64_f32out": _ragged("r6", "fp8_e4m3", "bf16", "f32", 64, 8, RAGGED, 6),
    "ragged_fp8_g1_d128_f16": _ragged("r7", "fp8_e4m3", "f16", "f16", 128, 1, RAGGED, 7),
    "ragged_fp8_g2_d128_f32": _ragged("r8", "fp8_e4m3", "f32", "f32", 128, 2, RAGGED, 8),
    "ragged_bf16_g8_d128_append": _ragged("r9", "bf16", "bf16", "bf16", 128, 8,
                                          [1, 16, 17, 200, 33, 48, 49], 9, hkv=3, append=True),
    # 8-bit mixed and int8 caches (K fp8 + V int8; int8 K with channel factors)
    "long_fp8k_int8v_small": scaled(WORKLOADS["long_fp8k_int8v"], num_seqs=2, len_range=(8192, 8192)),
    "long_int8_kchan_small": scaled(WORKLOADS["long_int8_kchan"], num_seqs=2, len_range=(8192, 8192)),
    "ragged_fp8k_int8v_g8_d64": _ragged("r10", "fp8_e4m3", "bf16", "bf16", 64, 8, RAGGED, 10, v="int8"),
    "ragged_fp8k_int8v_g1_d128_f16": _ragged("r11", "fp8_e4m3", "f16", "f16", 128, 1, RAGGED, 11, v="int8"),
    "ragged_int8_g4_d64_chan": _ragged("r12", "int8", "f16", "f16", 64, 4, RAGGED, 12, outliers=3),
    "ragged_int8_g2_d128_chan_append": _ragged("r13", "int8", "bf16", "bf16", 128, 2,
                                               [1, 16, 17, 200, 33, 48, 49], 13, hkv=3, append=True,
                                               outliers=5),
    "ragged_fp8k_int8v_g4_d128_chan_append": _ragged("r14", "fp8_e4m3", "bf16", "bf16", 128, 4,
                                                     [2, 15, 16, 64, 65, 300], 14, hkv=2, append=True,
                                                     v="int8", outliers=4),
    # attention-sink tokens in full-precision side tiles
    "ragged_int8_g8_d128_fpsinks4": _ragged("r15", "int8", "bf16", "bf16", 128, 8, RAGGED, 15, fp_sinks=4),
    "ragged_fp8_g2_d64_f32_fpsinks16": _ragged("r16", "fp8_e4m3", "f32", "f32", 64, 2, RAGGED, 16,
                                               fp_sinks=16),
    "ragged_fp8k_int8v_g4_d128_fpsinks3_append": _ragged("r17", "fp8_e4m3", "f16", "f16", 128, 4,
                                                         [1, 2, 3, 4, 17, 100], 17, hkv=2, append=True,
                                                         v="int8", outliers=2, fp_sinks=3),
    "long_fp8_fpsinks_small": scaled(WORKLOADS["long_fp8"], num_seqs=2, len_range=(8192, 8192), fp_sinks=4),
    # 8-bit caches on the matrix-core pass with an f32 query, or an f32 output
    "ragged_fp8_g4_d128_f32": _ragged("r19", "fp8_e4m3", "f32", "f32", 128, 4, RAGGED, 19),
    "ragged_fp8_g8_d128_bf16_f32out": _ragged("r20", "fp8_e4m3", "bf16", "f32", 128, 8, RAGGED, 20, hkv=3),
    # a table narrower than a workgroup's four waves (at most 3 blocks per
    # sequence), append carried: most waves of the matrix-core pass idle
    "narrow_table_f16_g8_d128_append": _ragged("r21", "f16", "f16", "f16", 128, 8, [1, 16, 17, 33, 2, 32],
                                               21, hkv=2, append=True),
    # one long sequence among short ones: the batch-size hint changes the split plan
    "one_long_many_short_f16": _ragged("r18", "f16", "f16", "f16", 128, 4, [8192] + [20, 3, 47, 16] * 4, 18),
    # V alone quantised, K kept in 16 bits (matrix-core and vector passes)
    "ragged_bf16k_fp8v_g4_d128": _ragged("r22", "bf16", "bf16", "bf16", 128, 4, RAGGED, 22, v="fp8_e4m3"),
    "ragged_f16k_int8v_g8_d128_append": _ragged("r23", "f16", "f16", "f16", 128, 8, [1, 16, 17, 200, 33, 48, 49],
                                                23, hkv=3, append=True, v="int8"),
    "ragged_f16k_fp8v_g2_d64": _ragged("r24", "f16", "f16", "f16", 64, 2, RAGGED, 24, v="fp8_e4m3"),
    "ragged_bf16k_int8v_g1_d128_vtok_append": _ragged("r25", "bf16", "bf16", "bf16", 128, 1,
                                                      [2, 15, 16, 64, 65, 300], 25, append=True, v="int8",
                                                      vtok=True),
    "ragged_f16k_fp8v_g4_d128_vtok": _ragged("r26", "f16", "f16", "f16", 128, 4, RAGGED, 26, v="fp8_e4m3",
                                             vtok=True),
    "long_bf16k_fp8v_small": scaled(WORKLOADS["long_bf16k_fp8v"], num_seqs=2, len_range=(8192, 8192)),
    # one scale per (token, KV head)
    "ragged_fp8_tok_g4_d128_append": _ragged("r27", "fp8_e4m3", "bf16", "bf16", 128, 4,
                                             [1, 16, 17, 200, 33, 48, 49], 27, append=True, ktok=True,
                                             vtok=True),
    "ragged_int8_tok_g8_d64_chan": _ragged("r28", "int8", "f16", "f16", 64, 8, RAGGED, 28, outliers=3,
                                           ktok=True, vtok=True),
    "ragged_fp8k_int8v_ktok_g8_d128": _ragged("r29", "fp8_e4m3", "bf16", "bf16", 128, 8, RAGGED, 29, hkv=3,
                                              v="int8", ktok=True),
    "ragged_fp8_vtok_g2_d128_f32": _ragged("r30", "fp8_e4m3", "f32", "f32", 128, 2, RAGGED, 30, vtok=True),
    "ragged_int8_tok_g4_d128_fpsinks4": _ragged("r31", "int8", "bf16", "bf16", 128, 4, RAGGED, 31, fp_sinks=4,
                                                ktok=True, vtok=True),
    "long_fp8_tok_small": scaled(WORKLOADS["long_fp8_tok"], num_seqs=2, len_range=(8192, 8192)),
    "ragged_int8_g8_d64_chan_ktok_append": _ragged("r32", "int8", "bf16", "bf16", 64, 8,
                                                   [1, 16, 17, 200, 33, 48, 49], 32, hkv=3, append=True,
                                                   outliers=3, ktok=True),
    "ragged_fp8_g8_d64_append_f32out": _ragged("r33", "fp8_e4m3", "f16", "f32", 64, 8, [5, 16, 17, 80, 33], 33,
                                               append=True),
    # more than 8 KV heads with an 8-bit cache and one partition (the KV head
    # is then the fastest workgroup index, as for 16-bit caches)
    "ragged_fp8_g1_d128_h12_append": _ragged("r34", "fp8_e4m3", "f16", "f16", 128, 1,
                                             [1, 16, 17, 200, 33, 48, 49], 51, hkv=12, append=True),
    "ragged_int8_g2_d64_h10": _ragged("r35", "int8", "bf16", "bf16", 64, 2, [1, 15, 16, 17, 31, 33, 100, 0, 64, 130],
                                      52, hkv=10),
    # the carried plain-copy append at the boundary where it moves behind the
    # first loads: lengths whose last piece gives the wave reading the new
    # token's block 1, 2 or exactly 3 steps (one partition), in the
    # matrix-core pass, the vector pass and with 4-byte elements
    "append_steps_f16_g8_d128": _ragged("r36", "f16", "f16", "f16", 128, 8, APPEND_STEPS, 53, append=True),
    "append_steps_bf16_g1_d128": _ragged("r37", "bf16", "bf16", "bf16", 128, 1, APPEND_STEPS, 54, hkv=3,
                                         append=True),
    "append_steps_f32_g2_d64": _ragged("r38", "f32", "f32", "f32", 64, 2, APPEND_STEPS, 55, append=True),
    # the same boundary for quantised rows (fp8, matrix-core pass), with
    # block scales and with per-token scales the new token sets
    "append_steps_fp8_g4_d128": _ragged("r39", "fp8_e4m3", "bf16", "bf16", 128, 4, APPEND_STEPS, 56, append=True),
    "append_steps_fp8_tok_g8_d128": _ragged("r40", "fp8_e4m3", "f16", "f16", 128, 8, APPEND_STEPS, 57,
                                            append=True, ktok=True, vtok=True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_matches_oracle(name):
    spec = SMALL[name]
    lay = build_layout(spec)
    say(f"[decode] {name}: B={spec.num_seqs} Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} "
        f"D={spec.head_dim} kv={spec.kv_dtype} lens={list(lay.context_lens[:12])}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    tol = TOL[spec.kv_dtype]
    for layer in range(spec.num_layers):
        out = _out(spec)
        run_step(xs, layer, spec, out)
        torch.cuda.synchronize()
        got = out_f64(out)
        ref = oracle_rows(host_layer(x, layer), lay, spec)
        assert np.isfinite(got).all()
        err = parity_err(got, ref, spec.out_dtype, tol)
        say(f"    layer {layer}: max|err| = {err:.3e} (tol {tol})")
        assert err <= tol
        zero = lay.context_lens == 0
        assert (got[zero] == 0).all()


WINDOWED = [
    # (case, window, sinks, partition_blocks)
    ("ragged_f16_g8_d128", 1, 0, 0),
    ("ragged_f16_g8_d128", 16, 0, 0),
    ("ragged_f16_g8_d128", 17, 4, 1),
    ("ragged_f16_g8_d128", 100, 20, 2),
    ("ragged_bf16_g4_d64", 33, 1, 0),
    ("ragged_bf16_g4_d64", 48, 64, 1),       # sinks overlap the window
    ("ragged_f32_g1_d64", 5, 3, 0),
    ("ragged_fp8_g2_d128_f32", 64, 16, 1),
    ("ragged_bf16_g8_d128_append", 30, 2, 0),
    ("long_fp8_small", 1024, 32, 0),
    ("llama3_8b_bf16_small", 700, 4, 0),
    ("ragged_fp8k_int8v_g8_d64", 40, 8, 1),
    ("long_int8_kchan_small", 2000, 16, 0),
    ("ragged_int8_g8_d128_fpsinks4", 30, 0, 0),
    ("ragged_fp8k_int8v_g4_d128_fpsinks3_append", 5, 0, 1),
    ("long_fp8_fpsinks_small", 1024, 0, 0),
]


@pytest.mark.parametrize("case,window,sinks", [(c, w, s) for c, w, s, pb in WINDOWED if pb == 0])
def test_balanced_split_with_window(case, window, sinks):
    """The batch-size hint counts whole lengths; with a window the kernels
    still attend only the window's blocks."""
    spec = SMALL[case]
    lay = build_layout(spec)
    say(f"[window+balanced] {case}: W={window} S={sinks} lens={list(lay.context_lens[:12])}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    out = _out(spec)
    run_step(xs, 0, spec, out, window=window, sinks=sinks, balanced=True)
    torch.cuda.synchronize()
    got = out_f64(out)
    ref = oracle_rows(host_layer(x, 0), lay, spec, window=window, sinks=sinks)
    err = parity_err(got, ref, spec.out_dtype, TOL[spec.kv_dtype])
    say(f"    max|err| = {err:.3e} (tol {TOL[spec.kv_dtype]})")
    assert np.isfinite(got).all() and err <= TOL[spec.kv_dtype]


@pytest.mark.parametrize("case,window,sinks,pb", WINDOWED)
def test_sliding_window_and_sinks(case, window, sinks, pb):
    spec = SMALL[case]
    lay = build_layout(spec)
    say(f"[window] {case}: W={window} S={sinks} partition_blocks={pb} lens={list(lay.context_lens[:12])}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    out = _out(spec)
    run_step(xs, 0, spec, out, partition_blocks=pb, window=window, sinks=sinks)
    torch.cuda.synchronize()
    got = out_f64(out)
    ref = oracle_rows(host_layer(x, 0), lay, spec, window=window, sinks=sinks)
    err = parity_err(got, ref, spec.out_dtype, TOL[spec.kv_dtype])
    say(f"    max|err| = {err:.3e} (tol {TOL[spec.kv_dtype]})")
    assert np.isfinite(got).all()
    assert err <= TOL[spec.kv_dtype]


@pytest.mark.parametrize("name", ["one_long_many_short_f16", "llama3_8b_bf16_small", "ragged_f16_g8_d128",
                                  "ragged_fp8_g2_d128_f32", "ragged_int8_g8_d128_fpsinks4", "long_fp8_small",
                                  "ragged_bf16_g4_d64", "ragged_f32_g1_d64", "ragged_fp8k_int8v_g8_d64",
                                  "ragged_int8_g4_d64_chan", "ragged_bf16_g8_d128_append"])
def test_balanced_plan_matches_oracle(name):
    """With the batch's block count passed, the split plan may change (for a
    light batch: pieces sized from the real total); the result still matches
    the oracle (sequences of length 0, 8-bit and mixed caches included)."""
    spec = SMALL[name]
    lay = build_layout(spec)
    say(f"[balanced] {name}: lens={list(lay.context_lens[:12])}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    out = _out(spec)
    run_step(xs, 0, spec, out, balanced=True)
    torch.cuda.synchronize()
    got = out_f64(out)
    ref = oracle_rows(host_layer(x, 0), lay, spec)
    err = parity_err(got, ref, spec.out_dtype, TOL[spec.kv_dtype])
    say(f"    max|err| = {err:.3e} (tol {TOL[spec.kv_dtype]})")
    assert np.isfinite(got).all() and err <= TOL[spec.kv_dtype]


# Shared-prefix groups: (case, group starts, shared blocks per group).  The
# ragged lengths are chosen so that every member extends past its group's
# shared blocks; sequences after the last start belong to no group.
GROUPED = {
    "prefix_one_group_f16_g1": ("mha13b_prefix_small", None, None),
    "prefix_groups_f16_g8_d128": (
        _ragged("p1", "f16", "f16", "f16", 128, 8, [300, 200, 180, 50, 260, 90, 40, 20, 600, 17, 1, 33],
                31, append=True),
        [0, 3, 3, 6, 9], [10, 0, 2, 1]),
    "prefix_groups_bf16_g4_d64": (
        _ragged("p2", "bf16", "bf16", "bf16", 64, 4, [700, 650, 601, 599, 1000, 70, 35, 17, 16],
                32, hkv=3),
        [0, 4, 6], [37, 2]),
    "prefix_two_chunks_f16_g8_d128": (       # 10 sequences x 8 heads = 80 query rows
        _ragged("p3", "f16", "f16", "f16", 128, 8, [400 + 37 * i for i in range(10)] + [5, 300],
                33, append=True),
        [0, 10], [23]),
    "prefix_groups_bf16_g2_d128_one_seq": (  # a one-sequence group and a 1-block group
        _ragged("p4", "bf16", "bf16", "bf16", 128, 2, [90, 130, 33, 34, 18, 257], 34, hkv=4),
        [0, 1, 2, 6], [5, 1, 1]),
    "prefix_groups_f16_g1_d64": (
        _ragged("p5", "f16", "f16", "f16", 64, 1, [130, 145, 161, 177, 193, 1], 35, hkv=5, append=True),
        [0, 5, 5], [8, 0]),
    # 8-bit caches: codes widened in the group pass, block scales on the scores and weights
    "prefix_groups_fp8_g1_d128": (
        _ragged("p6", "fp8_e4m3", "bf16", "bf16", 128, 1, [300, 200, 180, 50, 260, 90, 40, 20, 600, 17],
                36, hkv=5, append=True),
        [0, 3, 3, 7], [10, 0, 1]),
    "prefix_groups_int8_g4_d128": (
        _ragged("p7", "int8", "f16", "f16", 128, 4, [700, 650, 601, 599, 1000, 70, 35, 17, 16], 37, hkv=3),
        [0, 4, 6], [37, 2]),
    "prefix_two_chunks_fp8_g8_d128": (       # 10 sequences x 8 heads = 80 query rows
        _ragged("p8", "fp8_e4m3", "f16", "f16", 128, 8, [400 + 37 * i for i in range(10)] + [5, 300],
                38, append=True),
        [0, 10], [23]),
    "prefix_groups_int8_g2_d128_one_seq": (  # a one-sequence group and a 1-block group
        _ragged("p9", "int8", "bf16", "bf16", 128, 2, [90, 130, 33, 34, 18, 257], 39, hkv=4, append=True),
        [0, 1, 2, 6], [5, 1, 1]),
}


def _grouped_layout(case):
    src, starts, blocks = GROUPED[case]
    spec = SMALL[src] if isinstance(src, str) else src
    lay = build_layout(spec)
    if starts is not None:
        lay = share_prefixes(lay, starts, blocks)
    return spec, lay


@pytest.mark.parametrize("case", list(GROUPED))
def test_prefix_groups_match_oracle(case):
    """Shared prefixes read once per group (matrix-core pass) and merged with
    each sequence's own blocks: the oracle's attention, which knows nothing
    of groups, and the per-sequence path's result, to the same tolerance."""
    spec, lay = _grouped_layout(case)
    say(f"[groups] {case}: B={spec.num_seqs} g={spec.num_q_heads // spec.num_kv_heads} D={spec.head_dim} "
        f"starts={list(lay.group_starts)} blocks={list(lay.group_blocks)} lens={list(lay.context_lens)}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    plain = _out(spec)
    if not spec.append:
        run_step(xs, 0, spec, plain)                     # the per-sequence path
    grouped = _out(spec)
    run_step(xs, 0, spec, grouped, grouped=True)
    torch.cuda.synchronize()
    got = out_f64(grouped)
    ref = oracle_rows(host_layer(x, 0), lay, spec)
    tol = TOL[spec.kv_dtype]
    err = parity_err(got, ref, spec.out_dtype, tol)
    say(f"    max|err| = {err:.3e} (tol {tol})")
    assert np.isfinite(got).all() and err <= tol
    assert (got[lay.context_lens == 0] == 0).all()
    if not spec.append:                                  # same cache: the two paths agree
        assert max_err(got, out_f64(plain)) <= tol


@pytest.mark.parametrize("case", ["prefix_groups_f16_g8_d128", "prefix_groups_fp8_g1_d128"])
def test_prefix_groups_deterministic(case):
    """Two calls on the same inputs give bit-identical outputs (16-bit and
    8-bit caches)."""
    spec, lay = _grouped_layout(case)
    say(f"[groups] run-to-run: {case}")
    xs = _to_dev(make_host_inputs(lay))
    outs = []
    for i in range(3):
        o = _out(spec)
        run_step(xs, 0, spec, o, append=(i == 0), grouped=True)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[1], outs[2])


# Append and attention in one launch: (case, partition_blocks, window, sinks,
# skip); pb = -1 passes the batch's block count instead (the batch-size hint)
STEP_CASES = [
    ("tiny_f32", 0, 0, 0, None),
    ("tiny_f32", 2, 0, 0, 1),                      # split; sequence 1's token skipped
    ("tiny_f32", -1, 0, 0, 2),
    ("ragged_bf16_g8_d128_append", 0, 0, 0, None),
    ("ragged_bf16_g8_d128_append", 1, 0, 0, None),  # every block its own partition
    ("ragged_bf16_g8_d128_append", 0, 30, 2, None),
    ("ragged_bf16_g8_d128_append", -1, 0, 0, None),
    ("ragged_bf16_g8_d128_append", -1, 30, 2, 4),
    ("llama70b_f16_small", 0, 0, 0, None),
    ("mha13b_prefix_small", 0, 0, 0, 3),
    ("mha13b_prefix_small", -1, 0, 0, None),
    ("llama3_8b_bf16_small", 3, 700, 4, None),
    ("llama3_8b_bf16_small", -1, 0, 0, None),
    # the copying wave with 1, 2 or 3 steps (its copy moves behind the first
    # loads at 3), a skipped token among the latter
    ("append_steps_f16_g8_d128", 0, 0, 0, None),
    ("append_steps_bf16_g1_d128", 0, 0, 0, 0),
    ("append_steps_f32_g2_d64", 0, 0, 0, 2),
]


@pytest.mark.parametrize("case,pb,window,sinks,skip", STEP_CASES)
def test_fused_step_matches_append_then_attend(case, pb, window, sinks, skip):
    """pkv_paged_decode_step: the caches equal the oracle's append bit for
    bit, and the output the oracle's attention over them."""
    spec = SMALL[case]
    assert spec.append
    lay = build_layout(spec)
    say(f"[step] {case}: pb={pb} window={window} sinks={sinks} skip={skip} lens={list(lay.context_lens[:12])}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    slots = lay.slot_mapping.copy()
    if skip is not None:
        slots[skip] = -1
    sm = torch.from_numpy(slots).to(DEV)
    tol = TOL[spec.kv_dtype]
    for layer in range(spec.num_layers):
        out = _out(spec)
        total = int(((lay.context_lens.astype(np.int64) + 15) // 16).sum()) if pb < 0 else 0
        pkv.paged_decode_step(xs["k_new"][layer], xs["v_new"][layer], sm, xs["q"][layer], xs["k_cache"][layer],
                              xs["v_cache"][layer], xs["block_tables"], xs["context_lens"], spec.scale, out,
                              partition_blocks=max(pb, 0), window=window, sinks=sinks, total_blocks=total)
        torch.cuda.synchronize()
        h = host_layer(x, layer)
        kc, vc, _, _ = oracle_append(h, spec, slots)
        for name, ref in (("k_cache", kc), ("v_cache", vc)):
            got = host_storage(xs[name][layer])
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), (layer, name)
        keep = [b for b in range(spec.num_seqs) if b != skip]
        ref = oracle_attend(h, spec, kc, vc, None, None, lay.block_tables, lay.context_lens, seqs=keep,
                            window=window, sinks=sinks)
        got = out_f64(out)[keep]
        err = parity_err(got, ref, spec.out_dtype, tol)
        say(f"    layer {layer}: max|err| = {err:.3e} (tol {tol})")
        assert np.isfinite(got).all() and err <= tol


@pytest.mark.parametrize("case", ["prefix_one_group_f16_g1", "prefix_groups_f16_g8_d128",
                                  "prefix_two_chunks_f16_g8_d128", "prefix_groups_f16_g1_d64",
                                  "prefix_groups_fp8_g1_d128", "prefix_two_chunks_fp8_g8_d128",
                                  "prefix_groups_int8_g2_d128_one_seq"])
def test_fused_step_with_prefix_groups(case):
    """pkv_paged_decode_step_prefix (pkv_paged_decode_step_quant_prefix for
    8-bit caches, quantising on write with the blocks' scales): the append
    carried by the launch that reads shared prefixes once per group.  Every
    new token lies past its group's shared blocks.  Caches (and scales)
    equal the oracle's append bit for bit and the output the oracle's
    attention over them (the oracle knows nothing of groups)."""
    from gpu_common import group_args
    spec, lay = _grouped_layout(case)
    assert spec.append
    say(f"[step+groups] {case}: starts={list(lay.group_starts)} blocks={list(lay.group_blocks)} "
        f"lens={list(lay.context_lens)}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    out = _out(spec)
    kw = {}
    if spec.quantised:
        kw = dict(k_scales=xs["k_scales"][0], v_scales=xs["v_scales"][0])
    pkv.paged_decode_step(xs["k_new"][0], xs["v_new"][0], xs["slot_mapping"], xs["q"][0], xs["k_cache"][0],
                          xs["v_cache"][0], xs["block_tables"], xs["context_lens"], spec.scale, out,
                          **group_args(xs), **kw)
    torch.cuda.synchronize()
    h = host_layer(x, 0)
    kc, vc, ks, vs = oracle_append(h, spec, lay.slot_mapping)
    for name, ref in (("k_cache", kc), ("v_cache", vc), ("k_scales", ks), ("v_scales", vs)):
        if ref is None:
            continue
        assert np.array_equal(host_storage(xs[name][0]).view(np.uint8), ref.view(np.uint8)), name
    ref = oracle_attend(h, spec, kc, vc, ks, vs, lay.block_tables, lay.context_lens)
    tol = TOL[spec.kv_dtype]
    err = parity_err(out_f64(out), ref, spec.out_dtype, tol)
    say(f"    max|err| = {err:.3e} (tol {tol})")
    assert np.isfinite(out_f64(out)).all() and err <= tol


@pytest.mark.parametrize("case", ["split", "groups"])
def test_workspace_reused_across_calls(case):
    """One workspace serves several calls in a row (each call's pieces
    overwrite the previous call's): outputs are identical across the calls
    and equal the oracle's."""
    from gpu_common import group_args
    if case == "split":
        spec = SMALL["llama3_8b_bf16_small"]
        lay = build_layout(spec)
        kw = dict(partition_blocks=3)
    else:
        spec, lay = _grouped_layout("prefix_groups_f16_g8_d128")
        kw = {}
    say(f"[workspace reuse] {case}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    if case == "groups":
        kw.update(group_args(xs))
    first = _out(spec)
    dims = pkv.decode_dims(xs["q"][0], xs["k_cache"][0], xs["block_tables"], first,
                           kw.get("partition_blocks", 0), 0, 0, False, 0,
                           len(lay.group_blocks) if case == "groups" else 0, kw.get("prefix_max_seqs", 0),
                           kw.get("prefix_max_blocks", 0))
    need = pkv.decode_workspace_bytes(dims)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)    # NaN-filled partial rows
    if spec.append:
        pkv.kv_append(xs["k_new"][0], xs["v_new"][0], xs["slot_mapping"], xs["k_cache"][0], xs["v_cache"][0])
    outs = []
    for i in range(3):
        o = _out(spec)
        pkv.paged_decode_attn(xs["q"][0], xs["k_cache"][0], xs["v_cache"][0], xs["block_tables"],
                              xs["context_lens"], spec.scale, o, workspace=ws, **kw)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    ref = oracle_rows(host_layer(x, 0), lay, spec)
    err = parity_err(out_f64(outs[2]), ref, spec.out_dtype, TOL[spec.kv_dtype])
    say(f"    max|err| = {err:.3e}")
    assert err <= TOL[spec.kv_dtype]


QUANT_STEP_CASES = [
    ("long_fp8_small", 0, None),
    ("llama70b_fp8_small", 0, 1),
    ("ragged_int8_g2_d128_chan_append", 0, None),
    ("ragged_fp8k_int8v_g4_d128_chan_append", 2, 3),
    ("ragged_f16k_int8v_g8_d128_append", 0, None),
    ("ragged_bf16k_int8v_g1_d128_vtok_append", 1, None),
    ("ragged_fp8_tok_g4_d128_append", 0, 2),
    ("ragged_int8_g8_d64_chan_ktok_append", 0, None),
    ("ragged_fp8_g8_d64_append_f32out", 3, None),
    ("append_steps_fp8_g4_d128", 0, None),
    ("append_steps_fp8_tok_g8_d128", 0, 3),
]


@pytest.mark.parametrize("case,pb,skip", QUANT_STEP_CASES)
def test_fused_quant_step_matches_oracle(case, pb, skip):
    """pkv_paged_decode_step_quant: the new token quantised on write inside
    the attention launch (given block scales, or per-token scales the token
    sets; a 16-bit K copied): codes and scales equal the oracle's append bit
    for bit, the output the oracle's attention over them."""
    spec = SMALL[case]
    assert spec.append and spec.quantised
    lay = build_layout(spec)
    say(f"[step q8] {case}: pb={pb} skip={skip} k={spec.kv_dtype} v={spec.v_tag} "
        f"tok={spec.k_scale_tok},{spec.v_scale_tok} lens={list(lay.context_lens[:12])}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    slots = lay.slot_mapping.copy()
    if skip is not None:
        slots[skip] = -1
    sm = torch.from_numpy(slots).to(DEV)
    tol = TOL[spec.kv_dtype]
    for layer in range(spec.num_layers):
        out = _out(spec)
        kw = dict(v_scales=xs["v_scales"][layer])
        if spec.k_quantised:
            kw["k_scales"] = xs["k_scales"][layer]
        if "k_channel_scales" in xs:
            kw["k_channel_scales"] = xs["k_channel_scales"]
        pkv.paged_decode_step(xs["k_new"][layer], xs["v_new"][layer], sm, xs["q"][layer], xs["k_cache"][layer],
                              xs["v_cache"][layer], xs["block_tables"], xs["context_lens"], spec.scale, out,
                              partition_blocks=pb, **kw)
        torch.cuda.synchronize()
        h = host_layer(x, layer)
        kc, vc, ks, vs = oracle_append(h, spec, slots)
        for name, ref in (("k_cache", kc), ("v_cache", vc), ("k_scales", ks), ("v_scales", vs)):
            if ref is None:
                continue
            got = host_storage(xs[name][layer])
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), (layer, name)
        keep = [b for b in range(spec.num_seqs) if b != skip]
        ref = oracle_attend(h, spec, kc, vc, ks, vs, lay.block_tables, lay.context_lens, seqs=keep)
        got = out_f64(out)[keep]
        err = parity_err(got, ref, spec.out_dtype, tol)
        say(f"    layer {layer}: max|err| = {err:.3e} (tol {tol})")
        assert np.isfinite(got).all() and err <= tol


@pytest.mark.parametrize("pb", [1, 2, 3, 7])
def test_split_size_invariance(pb):
    say(f"[split] tiny_f32 partition_blocks={pb}")
    spec = WORKLOADS["tiny_f32"]
    lay = build_layout(spec)
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    whole = _out(spec)
    run_step(xs, 0, spec, whole, partition_blocks=1000)
    split = _out(spec)
    run_step(xs, 0, spec, split, partition_blocks=pb, append=False)
    torch.cuda.synchronize()
    ref = oracle_rows(host_layer(x, 0), lay, spec)
    assert max_err(out_f64(split), ref) <= 1e-5
    assert max_err(out_f64(split), out_f64(whole)) <= 2e-6


@pytest.mark.parametrize("pb", [1, 3])
def test_split_size_invariance_matrix_core(pb):
    """The matrix-core pass (fp8 cache, 8 query heads, head_dim 128, f32
    output): split into pieces of pb blocks and merged, or whole, the
    results agree to fp32 rounding and both match the oracle."""
    spec = SMALL["ragged_fp8_g8_d128_bf16_f32out"]
    say(f"[split] {spec.name} partition_blocks={pb}")
    lay = build_layout(spec)
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    whole = _out(spec)
    run_step(xs, 0, spec, whole, partition_blocks=1000)
    split = _out(spec)
    run_step(xs, 0, spec, split, partition_blocks=pb, append=False)
    torch.cuda.synchronize()
    ref = oracle_rows(host_layer(x, 0), lay, spec)
    assert max_err(out_f64(split), ref) <= 5e-2
    assert max_err(out_f64(split), out_f64(whole)) <= 1e-5


PRIVATE_COPY_CASES = {
    "mha13b_prefix_small": SMALL["mha13b_prefix_small"],
    # 64 query / 8 KV heads, head_dim 128: the matrix-core pass
    "gqa8_prefix_small": scaled(WORKLOADS["mha13b_prefix_f16"], name="gqa8_prefix_small", num_seqs=4,
                                num_q_heads=64, num_kv_heads=8),
}


@pytest.mark.parametrize("case", list(PRIVATE_COPY_CASES))
def test_shared_prefix_is_bit_identical_to_private_copies(case):
    """Same values, once shared (one block id in every table) and once
    copied into private blocks: the kernel must give bit-identical
    outputs."""
    spec = PRIVATE_COPY_CASES[case]
    say(f"[prefix] shared vs private copies: {case}")
    lay = build_layout(spec)
    x = make_host_inputs(lay)
    pb = spec.shared_prefix_tokens // 16
    kc, vc = x["k_cache"][0], x["v_cache"][0]
    NB = kc.shape[0]
    extra = (spec.num_seqs - 1) * pb
    kc2 = torch.cat([kc, torch.empty((extra,) + kc.shape[1:], dtype=kc.dtype)])
    vc2 = torch.cat([vc, torch.empty((extra,) + vc.shape[1:], dtype=vc.dtype)])
    tables2 = lay.block_tables.copy()
    nxt = NB
    for b in range(1, spec.num_seqs):
        for j in range(pb):
            src = lay.block_tables[b, j]
            kc2[nxt], vc2[nxt] = kc[src], vc[src]
            tables2[b, j] = nxt
            nxt += 1
    assert len(np.unique(tables2[tables2 >= 0])) == (tables2 >= 0).sum()
    outs = []
    for k_, v_, t_ in ((kc, vc, lay.block_tables), (kc2, vc2, tables2)):
        out = _out(spec)
        pkv.paged_decode_attn(x["q"][0].to(DEV), k_.to(DEV), v_.to(DEV),
                              torch.from_numpy(t_).to(DEV), x["context_lens"].to(DEV),
                              spec.scale, out)
        outs.append(out.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_deterministic_run_to_run():
    spec = SMALL["llama3_8b_bf16_small"]
    say("[determinism] two identical calls")
    lay = build_layout(spec)
    xs = _to_dev(make_host_inputs(lay))
    a, b = _out(spec), _out(spec)
    run_step(xs, 0, spec, a)
    run_step(xs, 0, spec, b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fp8_all_codes_decode_through_attention():
    """With one token, out = V: every e4m3 code (scale 1) comes out exactly
    as the OCP decoding (NaN codes as NaN)."""
    say("[fp8] 256 codes through a length-1 attention")
    D = 128
    codes = np.arange(256, dtype=np.uint8).reshape(2, D)
    vc = np.zeros((4, 1, 16, D), np.uint8)
    vc[1, 0, 0] = codes[0]
    vc[3, 0, 0] = codes[1]
    kc = np.full((4, 1, 16, D), 0x38, np.uint8)
    tables = np.array([[1], [3]], np.int32)
    lens = np.array([1, 1], np.int32)
    q = torch.randn((2, 1, D), device=DEV)
    out = torch.empty((2, 1, D), device=DEV)
    ones = torch.ones((4, 1), device=DEV)
    pkv.paged_decode_attn(q, torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
                          torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV), 0.1, out,
                          k_scales=ones, v_scales=ones)
    got = out.cpu().numpy()[:, 0, :].astype(np.float64)
    ref = oracle.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_block_ids_outside_pool_are_ignored():
    say("[bounds] table entries outside the pool")
    D, NB = 64, 3
    kc = torch.randn((NB, 1, 16, D), device=DEV)
    q = torch.randn((2, 4, D), device=DEV)
    tables = torch.tensor([[-7, NB + 1], [0, 1]], dtype=torch.int32, device=DEV)
    lens = torch.tensor([20, 20], dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    pkv.paged_decode_attn(q, kc, kc, tables, lens, 0.125, out)
    torch.cuda.synchronize()
    assert (out[0] == 0).all() and torch.isfinite(out[1]).all()


def test_lengths_past_the_table_are_clamped():
    """Positions past max_blocks_per_seq * 16 are not attended; a negative
    length is a zero row."""
    say("[bounds] lengths past the table width, negative lengths")
    spec = _ragged("clamp", "f16", "f16", "f16", 128, 4, [32, 32, 32, 20], 41)
    lay = build_layout(spec)
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    assert lay.block_tables.shape[1] == 2
    lens = torch.tensor([40, 33, -5, 20], dtype=torch.int32, device=DEV)   # table holds 32 positions
    out = _out(spec)
    pkv.paged_decode_attn(xs["q"][0], xs["k_cache"][0], xs["v_cache"][0], xs["block_tables"], lens,
                          spec.scale, out)
    torch.cuda.synchronize()
    got = out_f64(out)
    ref = oracle.paged_decode_attention(
        host_storage(x["q"][0]), host_storage(x["k_cache"][0]), host_storage(x["v_cache"][0]),
        lay.block_tables, np.array([32, 32, 0, 20]), spec.scale, q_tag="f16", kv_tag="f16")
    assert (got[2] == 0).all()
    assert parity_err(got, ref, "f16", TOL["f16"]) <= TOL["f16"]


@pytest.mark.parametrize("case", ["prefix_groups_f16_g8_d128", "prefix_two_chunks_fp8_g8_d128"])
def test_group_descriptors_out_of_range_do_not_fault(case):
    """Unsorted or out-of-range group starts and oversized block counts give
    undefined numbers but every access stays in bounds (the counts are
    clamped to the host bounds, the starts to [0, B]; with an 8-bit cache
    the block scales are read through the same clamped ids)."""
    spec, lay = _grouped_layout(case)
    say(f"[bounds] group descriptors out of range: {case}")
    xs = _to_dev(make_host_inputs(lay))
    width = lay.block_tables.shape[1]
    starts = torch.tensor([5, -3, 100, 2, 7], dtype=torch.int32, device=DEV)
    blocks = torch.tensor([1000, -4, width, 3], dtype=torch.int32, device=DEV)
    out = _out(spec)
    kw = dict(k_scales=xs["k_scales"][0], v_scales=xs["v_scales"][0]) if spec.quantised else {}
    pkv.paged_decode_attn(xs["q"][0], xs["k_cache"][0], xs["v_cache"][0], xs["block_tables"], xs["context_lens"],
                          spec.scale, out, prefix_group_starts=starts, prefix_group_blocks=blocks,
                          prefix_max_seqs=12, prefix_max_blocks=width, **kw)
    torch.cuda.synchronize()
    assert out.shape == (spec.num_seqs, spec.num_q_heads, spec.head_dim)


def test_hbm_read_probe_reads_every_word():
    """The bandwidth probe folds every 16-byte word into its workgroup's sink."""
    say("[probe] plain read fold")
    n16, W = 64 * 1024 + 5, 8
    x = torch.randint(0, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device=DEV)
    sink = torch.zeros(W, dtype=torch.int32, device=DEV)
    pkv.hbm_read_probe(x, sink)
    torch.cuda.synchronize()
    words = x.cpu().numpy().view(np.uint32).reshape(n16, 4)
    f = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    wg = np.arange(n16) // (-(-n16 // W))         # contiguous chunks of ceil(n16 / W) words
    exp = [int(np.bitwise_xor.reduce(f[wg == w])) for w in range(W)]
    assert sink.cpu().numpy().view(np.uint32).tolist() == exp


# --------------------------------------------------------------------------
# full-size workloads (the bench's launch configuration), sampled rows
# --------------------------------------------------------------------------

def _compact_rows(x, layer, lay, seqs):
    """Host copies of just the blocks `seqs` use, with tables remapped."""
    nblk = -(-lay.context_lens // 16)
    used = np.unique(np.concatenate([lay.block_tables[b, : nblk[b]] for b in seqs]))
    remap = {int(o): i for i, o in enumerate(used)}
    idx = torch.from_numpy(used.astype(np.int64)).to(DEV)
    h = {"q": host_storage(x["q"][layer]),
         "k_cache": host_storage(x["k_cache"][layer].index_select(0, idx)),
         "v_cache": host_storage(x["v_cache"][layer].index_select(0, idx))}
    for name in ("k_scales", "v_scales"):
        if name in x:
            h[name] = host_storage(x[name][layer].index_select(0, idx))
    if "k_channel_scales" in x:
        h["k_channel_scales"] = host_storage(x["k_channel_scales"])
    tables = np.full_like(lay.block_tables, -1)
    for b in seqs:
        tables[b, : nblk[b]] = [remap[int(o)] for o in lay.block_tables[b, : nblk[b]]]
    slots = None
    if lay.slot_mapping is not None:
        h["k_new"] = host_storage(x["k_new"][layer])
        h["v_new"] = host_storage(x["v_new"][layer])
        slots = np.full_like(lay.slot_mapping, -1)
        for b in seqs:
            s = int(lay.slot_mapping[b])
            slots[b] = remap[s // 16] * 16 + s % 16
    return h, tables, slots


@pytest.mark.parametrize("case,pb", [("ragged_f16_g8_d128", 1000), ("ragged_f16_g8_d128", 3),
                                     ("long_fp8_small", 64), ("ragged_bf16k_fp8v_g4_d128", 5),
                                     ("ragged_bf16k_int8v_g1_d128_vtok_append", 4)])
def test_paged_read_probe_reads_exactly_the_attended_tiles(case, pb):
    """The access-pattern probe reads, per workgroup (sequence, KV head,
    partition), every 32-bit word of the K and V rows that hold a token in
    the blocks that partition covers and nothing else: its sink equals the
    XOR of exactly those words, computed on the host."""
    spec = SMALL[case]
    lay = build_layout(spec)
    say(f"[probe] {case}: pb={pb} lens={list(lay.context_lens[:12])}")
    x = make_host_inputs(lay)
    xs = _to_dev(x)
    out = _out(spec)
    dims = pkv.decode_dims(xs["q"][0], xs["k_cache"][0], xs["block_tables"], out, partition_blocks=pb)
    P = pkv.decode_num_partitions(dims)
    sink = torch.zeros(spec.num_seqs * spec.num_kv_heads * P, dtype=torch.int32, device=DEV)
    pkv.paged_read_probe(xs["k_cache"][0], xs["v_cache"][0], xs["block_tables"], xs["context_lens"], dims, sink)
    torch.cuda.synchronize()
    kw = x["k_cache"][0].contiguous().view(torch.int32).numpy()
    vw = x["v_cache"][0].contiguous().view(torch.int32).numpy()
    pbk = min(pb, lay.max_blocks_per_seq)           # the plan's piece size
    want = np.zeros_like(sink.cpu().numpy())
    for b in range(spec.num_seqs):
        natt = -(-int(lay.context_lens[b]) // 16)
        n = min(-(-natt // pbk), P) if natt else 0
        per = -(-natt // n) if n else 0
        for h in range(spec.num_kv_heads):
            for p in range(P):
                acc = np.int32(0)
                for j in range(p * per, min(p * per + per, natt)):
                    blk = int(lay.block_tables[b, j])
                    nv = min(16, int(lay.context_lens[b]) - 16 * j)     # rows holding a token
                    acc ^= (np.bitwise_xor.reduce(kw[blk, h, :nv].ravel()) ^
                            np.bitwise_xor.reduce(vw[blk, h, :nv].ravel()))
                want[(b * spec.num_kv_heads + h) * P + p] = acc
    assert np.array_equal(sink.cpu().numpy(), want)


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "mha13b_prefix_f16", "mha13b_prefix_f16:grouped", "long_fp8",
                                  "llama70b_f16_80l", "llama70b_fp8_80l", "long_fp8k_int8v", "long_int8_kchan",
                                  "long_bf16k_fp8v", "long_fp8_tok", "mha13b_prefix_bf16:grouped",
                                  "mha13b_prefix_fp8:grouped"])
def test_full_size_sampled_rows(name):
    name, _, mode = name.partition(":")
    grouped = mode == "grouped"
    spec = WORKLOADS[name]
    lay = build_layout(spec)
    say(f"[full] {name}: B={spec.num_seqs} layers={spec.num_layers} blocks={lay.num_blocks} "
        f"partitions={pkv.decode_num_partitions(pkv.DecodeDims(spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, 16, lay.num_blocks, lay.max_blocks_per_seq, 0, 0, 0, 0))}")
    x = make_device_inputs(lay, DEV)
    rng = np.random.default_rng(spec.seed)
    layers = sorted({0, spec.num_layers // 2, spec.num_layers - 1})
    seqs = sorted(rng.choice(spec.num_seqs, size=min(3, spec.num_seqs), replace=False).tolist())
    heads = sorted(rng.choice(spec.num_q_heads, size=min(4, spec.num_q_heads), replace=False).tolist())
    snaps = {l: _compact_rows(x, l, lay, seqs) for l in layers}        # before the step writes
    outs = {}
    for layer in range(spec.num_layers):                               # the whole step
        out = _out(spec)
        run_step(x, layer, spec, out, grouped=grouped)
        if layer in snaps:
            outs[layer] = out
    torch.cuda.synchronize()
    tol = TOL[spec.kv_dtype]
    for layer in layers:
        h, tables, slots = snaps[layer]
        kc, vc, ks, vs = oracle_append(h, spec, slots)
        ref = oracle_attend(h, spec, kc, vc, ks, vs, tables, lay.context_lens, seqs=seqs, q_heads=heads)
        got = out_f64(outs[layer])[seqs][:, heads]
        err = parity_err(got, ref, spec.out_dtype, tol)
        say(f"    layer {layer} seqs {seqs} heads {heads}: max|err| = {err:.3e} (tol {tol})")
        assert err <= tol
        assert torch.isfinite(outs[layer].float()).all()
    del x
    torch.cuda.empty_cache()
