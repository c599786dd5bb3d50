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


# --------------------------------------------------------------------------
# FP8 quantise-on-write
# --------------------------------------------------------------------------

from oracle import kv_append_fp8, decode_e4m3fn


def _fp8_case(seed=3, T=6, H=2, D=8, NB=5):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x70, size=(NB, H, BS, D)).astype(np.uint8)
    scales = rng.uniform(0.01, 0.1, size=(NB, H)).astype(np.float32)
    x = (rng.standard_normal((T, H, D)) * 3).astype(np.float32)
    return codes, scales, x


def test_fp8_append_given_scales_matches_torch_cast():
    """Codes = torch's float8_e4m3fn cast of the clamped fp32 quotient."""
    codes, scales, x = _fp8_case()
    slots = np.array([0, 17, 33, -1, 50, 79])
    out, sc = kv_append_fp8(codes, scales, x, slots, first_write=False)
    assert np.array_equal(sc, scales)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        q = np.clip(x[t] / scales[s // BS][:, None], -448, 448).astype(np.float32)
        ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(out[s // BS, :, s % BS, :], ref)
    # untouched elsewhere
    mask = np.ones(codes.shape, bool)
    for s in slots[slots >= 0]:
        mask[s // BS, :, s % BS, :] = False
    assert np.array_equal(out[mask], codes[mask])


def test_fp8_append_first_write_sets_scale_then_saturates():
    codes, scales, x = _fp8_case(T=3)
    x[1] = x[0] * 4                     # a later token of the same block, 4x larger
    slots = np.array([32, 33, 48])      # block 2 starts with token 0; block 3 with token 2
    out, sc = kv_append_fp8(codes, scales, x, slots, first_write=True)
    for t, blk in ((0, 2), (2, 3)):
        amax = np.abs(x[t]).max(axis=1)
        assert np.array_equal(sc[blk], (amax / np.float32(448)).astype(np.float32))
        row = decode_e4m3fn(out[blk, :, 0 if t == 0 else 0, :])
        assert np.array_equal(np.abs(row).max(axis=1), [448.0, 448.0])
    # token 1 reused block 2's scale and saturated where it exceeded 448 * scale
    dec = decode_e4m3fn(out[2, :, 1, :])
    big = np.abs(x[1]) / sc[2][:, None] > 448
    assert big.any() and np.all(np.abs(dec[big]) == 448.0)
    assert np.array_equal(sc[[0, 1, 4]], scales[[0, 1, 4]])


def test_fp8_append_exact_values_round_trip():
    """x = decode(c) * 2^k is stored as c exactly (power-of-two scales)."""
    rng = np.random.default_rng(4)
    c = rng.integers(0, 0x7F, size=(2, 1, 8)).astype(np.uint8)
    c[c == 0x7F] = 0
    scales = np.array([[0.25], [8.0]], np.float32)
    x = (decode_e4m3fn(c)[:, :, :] * scales[[0, 1]][:, :, None]).astype(np.float32)
    codes = np.zeros((2, 1, BS, 8), np.uint8)
    out, _ = kv_append_fp8(codes, scales, x, np.array([3, 16 + 5]), first_write=False)
    assert np.array_equal(out[0, :, 3, :], c[0]) and np.array_equal(out[1, :, 5, :], c[1])


def test_fp8_append_zero_token_first_write_scale_is_one():
    codes, scales, x = _fp8_case(T=1)
    x[:] = 0
    out, sc = kv_append_fp8(codes, scales, x, np.array([16]), first_write=True)
    assert np.all(sc[1] == 1.0) and np.all(out[1, :, 0, :] == 0)


# --------------------------------------------------------------------------
# INT8 quantise-on-write, per-channel factors
# --------------------------------------------------------------------------

from oracle import kv_append_int8, kv_append_quant


def _nearest_int8_brute(q):
    """Nearest of -127..127 to each fp32 value, ties to the even code, by
    scanning every candidate (NaN -> 0)."""
    cand = np.arange(-127, 128, dtype=np.float64)
    out = np.zeros(q.shape, np.int8)
    for idx, v in np.ndenumerate(q.astype(np.float64)):
        if np.isnan(v):
            continue
        dist = np.abs(cand - v)
        best = np.flatnonzero(dist == dist.min())
        if len(best) == 2:                       # a tie: the even code wins
            best = best[(cand[best] % 2) == 0]
        out[idx] = int(cand[best[0]])
    return out


def _int8_case(seed=5, T=6, H=2, D=8, NB=5):
    rng = np.random.default_rng(seed)
    codes = rng.integers(-127, 128, size=(NB, H, BS, D)).astype(np.int8)
    scales = rng.uniform(0.01, 0.1, size=(NB, H)).astype(np.float32)
    x = (rng.standard_normal((T, H, D)) * 3).astype(np.float32)
    return codes, scales, x


def test_int8_append_given_scales_is_nearest_code():
    codes, scales, x = _int8_case()
    x[0, 0, :4] = np.array([0.5, 1.5, -2.5, 126.5], np.float32) * scales[0, 0]   # halves
    x[1, 1, :3] = np.array([1000.0, -1000.0, np.nan], np.float32)               # saturate, NaN
    slots = np.array([0, 17, 33, -1, 50, 79])
    out, sc = kv_append_int8(codes, scales, x, slots, first_write=False)
    assert np.array_equal(sc, scales)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        q = np.clip(x[t] / scales[s // BS][:, None], -127, 127).astype(np.float32)
        assert np.array_equal(out[s // BS, :, s % BS, :], _nearest_int8_brute(q))
    assert list(out[0, 0, 0, :4]) == [0, 2, -2, 126]
    assert list(out[1, 1, 1, :3]) == [127, -127, 0]
    mask = np.ones(codes.shape, bool)
    for s in slots[slots >= 0]:
        mask[s // BS, :, s % BS, :] = False
    assert np.array_equal(out[mask], codes[mask])


def test_int8_append_first_write_sets_scale_then_saturates():
    codes, scales, x = _int8_case(T=3)
    x[1] = x[0] * 4
    slots = np.array([32, 33, 48])
    out, sc = kv_append_int8(codes, scales, x, slots, first_write=True)
    for t, blk in ((0, 2), (2, 3)):
        amax = np.abs(x[t]).max(axis=1)
        assert np.array_equal(sc[blk], (amax / np.float32(127)).astype(np.float32))
        assert np.array_equal(np.abs(out[blk, :, 0, :].astype(int)).max(axis=1), [127, 127])
    big = np.abs(x[1]) / sc[2][:, None] > 127.5
    assert big.any() and np.all(np.abs(out[2, :, 1, :][big].astype(int)) == 127)
    # dequantisation error of the unsaturated elements is at most half a step
    ok = ~big
    err = np.abs(out[2, :, 1, :].astype(np.float64) * sc[2][:, None] - x[1])
    assert np.all(err[ok] <= 0.5 * np.broadcast_to(sc[2][:, None], err.shape)[ok] * (1 + 1e-6))
    assert np.array_equal(sc[[0, 1, 4]], scales[[0, 1, 4]])


def test_int8_append_exact_values_round_trip_and_zero_row():
    rng = np.random.default_rng(6)
    c = rng.integers(-127, 128, size=(2, 1, 8)).astype(np.int8)
    scales = np.array([[0.25], [8.0]], np.float32)
    x = (c.astype(np.float32) * scales[:, :, None]).astype(np.float32)
    out, _ = kv_append_int8(np.zeros((2, 1, BS, 8), np.int8), scales, x, np.array([3, 21]),
                            first_write=False)
    assert np.array_equal(out[0, :, 3, :], c[0]) and np.array_equal(out[1, :, 5, :], c[1])
    z = np.zeros((1, 1, 8), np.float32)
    out, sc = kv_append_int8(np.ones((2, 1, BS, 8), np.int8), scales, z, np.array([16]), first_write=True)
    assert sc[1, 0] == 1.0 and np.all(out[1, :, 0, :] == 0)


@pytest.mark.parametrize("code", ["fp8_e4m3", "int8"])
def test_channel_scales_divide_before_quantising(code):
    """Power-of-two channel factors divide exactly, so appending x with factors
    c equals appending x / c without them; unit factors change nothing."""
    rng = np.random.default_rng(7)
    H, D, NB = 2, 8, 3
    dt = np.uint8 if code == "fp8_e4m3" else np.int8
    codes = np.zeros((NB, H, BS, D), dt)
    scales = np.ones((NB, H), np.float32)
    c = (2.0 ** rng.integers(-3, 5, size=(H, D))).astype(np.float32)
    x = (rng.standard_normal((4, H, D)) * 5 * c).astype(np.float32)
    slots = np.array([16, 17, 32, 2])
    for fw in (False, True):
        got = kv_append_quant(codes, scales, x, slots, code=code, first_write=fw, channel_scales=c)
        ref = kv_append_quant(codes, scales, x / c, slots, code=code, first_write=fw)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        one = kv_append_quant(codes, scales, x, slots, code=code, first_write=fw,
                              channel_scales=np.ones((H, D), np.float32))
        plain = kv_append_quant(codes, scales, x, slots, code=code, first_write=fw)
        assert np.array_equal(one[0], plain[0]) and np.array_equal(one[1], plain[1])
    # an outlier channel no longer flattens the others: every channel of a
    # first-written int8 row spans the code range it has
    x2 = rng.standard_normal((1, H, D)).astype(np.float32)
    x2[0, :, 3] *= 64
    cs = np.ones((H, D), np.float32); cs[:, 3] = 64
    out_c, _ = kv_append_int8(np.zeros((NB, H, BS, D), np.int8), scales, x2, np.array([0]),
                              first_write=True, channel_scales=cs)
    out_n, _ = kv_append_int8(np.zeros((NB, H, BS, D), np.int8), scales, x2, np.array([0]),
                              first_write=True)
    others = [d for d in range(D) if d != 3]
    assert (np.abs(out_c[0, :, 0, others].astype(int)).max() >
            4 * np.abs(out_n[0, :, 0, others].astype(int)).max())


# --------------------------------------------------------------------------
# per-token scales ("KV Cache from first principles" 5.2: per-token granularity)
# --------------------------------------------------------------------------

def _token_case(code, seed=7, T=5, H=2, D=8, NB=4):
    rng = np.random.default_rng(seed)
    if code == "fp8_e4m3":
        codes = rng.integers(0, 0x70, size=(NB, H, BS, D)).astype(np.uint8)
    else:
        codes = rng.integers(-127, 128, size=(NB, H, BS, D)).astype(np.int8)
    scales = rng.uniform(0.01, 0.1, size=(NB, H, BS)).astype(np.float32)
    x = (rng.standard_normal((T, H, D)) * 3).astype(np.float32)
    x[1] *= 50                                     # one token far larger than the others
    return codes, scales, x


@pytest.mark.parametrize("code", ["fp8_e4m3", "int8"])
def test_per_token_append_scales_each_token_by_its_own_row(code):
    """Each written token's (slot, head) scale is its row's max |x| / QMAX;
    its largest element lands exactly on +-QMAX; codes are torch's float8
    cast (fp8) or the brute-force nearest integer (int8) of the fp32
    quotient; no other slot or scale changes."""
    codes, scales, x = _token_case(code)
    slots = np.array([0, 17, 33, -1, 63])
    out, sc = kv_append_quant(codes, scales, x, slots, code=code, first_write=False, granularity="token")
    qmax = np.float32(448 if code == "fp8_e4m3" else 127)
    touched = np.zeros(scales.shape, bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = s // BS, s % BS
        amax = np.abs(x[t]).max(axis=1)
        assert np.array_equal(sc[blk, :, off], (amax / qmax).astype(np.float32))
        touched[blk, :, off] = True
        q = np.clip(x[t] / sc[blk, :, off][:, None], -qmax, qmax).astype(np.float32)
        got = out[blk, :, off, :]
        if code == "fp8_e4m3":
            ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(got, ref)
            peak = np.abs(decode_e4m3fn(got)).max(axis=1)
        else:
            assert np.array_equal(got, _nearest_int8_brute(q))
            peak = np.abs(got.astype(np.float64)).max(axis=1)
        assert np.array_equal(peak, [float(qmax)] * x.shape[1])
    assert np.array_equal(sc[~touched], scales[~touched])
    mask = np.ones(codes.shape, bool)
    for s in slots[slots >= 0]:
        mask[s // BS, :, s % BS, :] = False
    assert np.array_equal(out[mask], codes[mask])


def test_per_token_append_round_trips_and_rejects_bad_calls():
    """A row that is a code vector times a power of two with its largest
    code at +-QMAX comes back as the same codes and that scale; a zero row
    gets scale 1; first-write mode and block-shaped scales are refused."""
    rng = np.random.default_rng(8)
    c = rng.integers(-127, 128, size=(1, 2, 8)).astype(np.int8)
    c[0, :, 0] = [127, -127]
    x = (c.astype(np.float32) * np.float32(0.125))
    codes = np.zeros((2, 2, BS, 8), np.int8)
    scales = np.zeros((2, 2, BS), np.float32)
    out, sc = kv_append_quant(codes, scales, x, np.array([21]), code="int8", first_write=False,
                              granularity="token")
    assert np.array_equal(out[1, :, 5, :], c[0]) and np.array_equal(sc[1, :, 5], [0.125, 0.125])
    out, sc = kv_append_quant(codes, scales, np.zeros((1, 2, 8), np.float32), np.array([3]), code="int8",
                              first_write=False, granularity="token")
    assert np.all(sc[0, :, 3] == 1.0) and np.all(out[0, :, 3, :] == 0)
    with pytest.raises(ValueError):
        kv_append_quant(codes, scales, x, np.array([3]), code="int8", first_write=True, granularity="token")
    with pytest.raises(ValueError):
        kv_append_quant(codes, scales[:, :, 0], x, np.array([3]), code="int8", first_write=False,
                        granularity="token")
    with pytest.raises(ValueError):
        kv_append_quant(codes, scales, x, np.array([3]), code="int8", first_write=False)
