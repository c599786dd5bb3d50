"""The C ABI on a machine without a GPU: exports, status codes, sizing.

Every call here fails validation (or needs no launch), so nothing reaches
the device.
"""

import ctypes
import os
import re

import pytest
import torch

import paged_kv_cache_56_amd as pkv
from paged_kv_cache_56_amd import DecodeDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _declared():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"^PKV_API\b[^;(]*?\b(pkv_\w+)\s*\(", text, flags=re.M)
    return names


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 7
    lib = pkv.load_library()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pkv_version() == 181


def _dims(**kw):
    base = dict(num_seqs=64, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                num_blocks=16384, max_blocks_per_seq=256, q_dtype=1, kv_dtype=1, out_dtype=1,
                partition_blocks=0)
    base.update(kw)
    return DecodeDims(**base)


def _attn(dims, q=FAKE, ws=None, ws_bytes=0):
    lib = pkv.load_library()
    return lib.pkv_paged_decode_attn(q, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.088), FAKE,
                                     ctypes.byref(dims), ws, ws_bytes, None)


def _attn_fp8(dims, ks=FAKE, vs=FAKE):
    lib = pkv.load_library()
    return lib.pkv_paged_decode_attn_fp8(FAKE, FAKE, FAKE, ks, vs, FAKE, FAKE, ctypes.c_float(0.088),
                                         FAKE, ctypes.byref(dims), None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(block_size=8), -2),
    (dict(num_q_heads=60), -2),            # Hq % Hkv
    (dict(num_q_heads=128), -2),           # g = 16
    (dict(head_dim=96), -2),
    (dict(num_seqs=0), -2),
    (dict(max_blocks_per_seq=0), -2),
    (dict(num_blocks=-1), -2),
    (dict(partition_blocks=-3), -2),
    (dict(window=-1), -2),
    (dict(window=64, sinks=-1), -2),
    (dict(q_dtype=2), -3),                 # q bf16, cache f16
    (dict(out_dtype=0), -3),
    (dict(kv_dtype=3, q_dtype=3, out_dtype=3), -3),  # fp8 through the non-fp8 entry
    (dict(q_dtype=7), -3),
])
def test_attn_status_codes(kw, status):
    assert _attn(_dims(**kw)) == status


def test_attn_null_and_workspace():
    assert _attn(_dims(), q=None) == -1
    d = _dims(num_seqs=16)                 # 16 x 8 units -> split in four
    need = pkv.decode_workspace_bytes(d)
    assert need == 16 * 64 * 4 * (128 + 2) * 4
    assert _attn(d, ws=None, ws_bytes=0) == -4
    assert _attn(d, ws=FAKE, ws_bytes=need - 1) == -4
    assert _attn(_dims(num_seqs=16), ws=FAKE, ws_bytes=need - 4) == -4
    assert pkv.decode_workspace_bytes(_dims()) == 0     # 512 units: no split


def test_fp8_status_codes():
    ok = dict(kv_dtype=3, q_dtype=2, out_dtype=2, num_q_heads=32, max_blocks_per_seq=16)
    assert _attn_fp8(_dims(**ok), ks=None) == -1
    assert _attn_fp8(_dims(**ok), vs=None) == -1
    assert _attn_fp8(_dims(**dict(ok, kv_dtype=1))) == -3
    assert _attn_fp8(_dims(**dict(ok, q_dtype=3))) == -3
    assert _attn_fp8(_dims(**dict(ok, out_dtype=1))) == -3        # bf16 q, f16 out


def _attn_quant(dims, v_dtype, ks=FAKE, vs=FAKE, q=FAKE, sink=None, ntiles=0, params=True):
    lib = pkv.load_library()
    qp = pkv.QuantParams(ks and ks.value, vs and vs.value, None, v_dtype, sink, sink, sink, ntiles)
    return lib.pkv_paged_decode_attn_quant(q, FAKE, FAKE, ctypes.byref(qp) if params else None, FAKE,
                                           FAKE, ctypes.c_float(0.088), FAKE, ctypes.byref(dims), None,
                                           0, None)


def test_quant_status_codes():
    """Pairs outside (fp8, fp8), (fp8, int8), (int8, int8), or with a query /
    output pairing those pairs do not take, are refused before any launch."""
    ok = dict(q_dtype=2, out_dtype=2, num_q_heads=32, max_blocks_per_seq=16)
    for k, v in ((4, 3), (1, 4), (3, 1), (4, 2)):          # int8 K + fp8 V, f16 K, ...
        assert _attn_quant(_dims(**dict(ok, kv_dtype=k)), v) == -3, (k, v)
    assert _attn_quant(_dims(**dict(ok, kv_dtype=3, out_dtype=0)), 4) == -3    # mixed, f32 out
    assert _attn_quant(_dims(**dict(ok, kv_dtype=4, q_dtype=0, out_dtype=0)), 4) == -3
    assert _attn_quant(_dims(**dict(ok, kv_dtype=4, q_dtype=4, out_dtype=4)), 4) == -3
    assert _attn_quant(_dims(**dict(ok, kv_dtype=3)), 4, ks=None) == -1
    assert _attn_quant(_dims(**dict(ok, kv_dtype=4)), 4, vs=None) == -1
    assert _attn_quant(_dims(**dict(ok, kv_dtype=4)), 4, q=None) == -1
    assert _attn_quant(_dims(**dict(ok, kv_dtype=4, head_dim=96)), 4) == -2
    assert _attn_quant(_dims(**dict(ok, kv_dtype=4)), 4, params=False) == -1
    # int8 through the other entry points
    assert _attn(_dims(kv_dtype=4, q_dtype=4, out_dtype=4)) == -3
    assert _attn_fp8(_dims(kv_dtype=4, q_dtype=2, out_dtype=2)) == -3


def test_sink_tile_status_codes_and_workspace():
    ok = dict(kv_dtype=4, q_dtype=2, out_dtype=2, num_q_heads=32, max_blocks_per_seq=16, sinks=4,
              sink_tiles=1)
    assert _attn_quant(_dims(**ok), 4) == -1                          # tiles missing
    assert _attn_quant(_dims(**ok), 4, sink=FAKE.value, ntiles=0) == -2
    assert _attn_quant(_dims(**dict(ok, sinks=0)), 4, sink=FAKE.value, ntiles=3) == -2
    assert _attn_quant(_dims(**dict(ok, sinks=17)), 4, sink=FAKE.value, ntiles=3) == -2
    assert _attn_quant(_dims(**dict(ok, sink_tiles=2)), 4, sink=FAKE.value, ntiles=3) == -2
    assert _attn(_dims(sinks=4, sink_tiles=1)) == -2                  # not on the 16-bit entry
    assert _attn_fp8(_dims(**dict(ok, kv_dtype=3))) == -2             # nor on the fp8 one
    # always split (the merge kernel attends the sink tiles), even when P = 1
    d = _dims(**ok)
    assert pkv.decode_num_partitions(d) == 1
    assert pkv.decode_workspace_bytes(d) == 64 * 32 * 1 * (128 + 2) * 4
    assert _attn_quant(d, 4, sink=FAKE.value, ntiles=3) == -4        # no workspace given


def _attn_prefix(dims, starts=FAKE, blocks=FAKE, ws=None, ws_bytes=0):
    lib = pkv.load_library()
    return lib.pkv_paged_decode_attn_prefix(FAKE, FAKE, FAKE, starts, blocks, FAKE, FAKE,
                                            ctypes.c_float(0.088), FAKE, ctypes.byref(dims), ws,
                                            ws_bytes, None)


def test_prefix_group_status_codes_and_plan():
    # the MHA prefix batch: 64 sequences x 40 heads, one group sharing 75 blocks
    ok = dict(num_seqs=64, num_q_heads=40, num_kv_heads=40, max_blocks_per_seq=100,
              prefix_groups=1, prefix_max_seqs=64, prefix_max_blocks=75)
    d = _dims(**ok)
    # per-sequence pass: 1 piece; group pass: pieces of at least 32 blocks
    # -> 3 pieces of 25; every row gets 1 + 3 workspace slots
    assert pkv.decode_num_partitions(d) == 1
    assert pkv.decode_workspace_bytes(d) == 64 * 40 * (1 + 3) * (128 + 2) * 4
    assert _attn_prefix(d) == -4                                   # valid, but no workspace
    assert _attn_prefix(d, starts=None) == -1
    assert _attn_prefix(d, blocks=None) == -1
    for bad in (dict(prefix_groups=-1), dict(prefix_max_seqs=0), dict(prefix_max_blocks=101),
                dict(prefix_max_blocks=-1), dict(window=256), dict(sinks=4, sink_tiles=1),
                dict(prefix_groups=65535, prefix_max_seqs=65)):    # grid z: 65535 x 2 chunks
        assert _attn_prefix(_dims(**dict(ok, **bad))) == -2, bad
    for dt in (dict(q_dtype=0, kv_dtype=0, out_dtype=0), dict(kv_dtype=3, q_dtype=2, out_dtype=2),
               dict(kv_dtype=2)):
        assert _attn_prefix(_dims(**dict(ok, **dt))) == -3, dt
    # groups only through their own entry point
    assert _attn(d) == -2
    assert _attn_fp8(_dims(**dict(ok, kv_dtype=3, q_dtype=2, out_dtype=2))) == -2
    assert _attn_quant(_dims(**dict(ok, kv_dtype=4, q_dtype=2, out_dtype=2)), 4) == -2
    # no groups: the entry point behaves like pkv_paged_decode_attn (no split here)
    d0 = _dims(**dict(ok, prefix_groups=0))
    assert pkv.decode_workspace_bytes(d0) == 0
    # more query rows than one chunk: the group pass needs no more slots
    d8 = _dims(num_seqs=64, num_q_heads=64, num_kv_heads=8, max_blocks_per_seq=256,
               prefix_groups=2, prefix_max_seqs=40, prefix_max_blocks=200)
    # group pass: 2 groups x 8 heads x 5 chunks = 80 units -> ~256 workgroups
    # would take 4 pieces of 50 blocks (above the 32-block floor)
    assert pkv.decode_workspace_bytes(d8) == 64 * 64 * (1 + 4) * (128 + 2) * 4


def _step(dims, k_new=FAKE, v_new=FAKE, slots=FAKE, ws=None, ws_bytes=0):
    lib = pkv.load_library()
    return lib.pkv_paged_decode_step(k_new, v_new, slots, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.088),
                                     FAKE, ctypes.byref(dims), ws, ws_bytes, None)


def test_fused_step_status_codes():
    d = _dims(num_seqs=16)                       # 16 x 8 units -> 4 partitions: needs a workspace
    assert pkv.decode_num_partitions(d) == 4
    assert _step(d) == -4
    assert _step(d, k_new=None) == -1
    assert _step(d, slots=None) == -1
    assert _step(_dims(kv_dtype=3, q_dtype=2, out_dtype=2)) == -3          # 8-bit caches: separate calls
    assert _step(_dims(kv_dtype=4, q_dtype=2, out_dtype=2)) == -3
    assert _step(_dims(kv_dtype=1, q_dtype=2, out_dtype=2)) == -3          # q, caches, out of one type
    assert _step(_dims(sinks=4, sink_tiles=1)) == -2
    assert _step(_dims(prefix_groups=1, prefix_max_seqs=4, prefix_max_blocks=8)) == -2
    assert _step(_dims(block_size=8)) == -2


def test_append_quant_status_codes():
    lib = pkv.load_library()
    call = lambda *a: lib.pkv_kv_append_quant(*a, None)
    # x, slots, cache, scales, chan, T, Hkv, D, NB, bs, src, cache_dtype, mode
    assert call(FAKE, FAKE, FAKE, FAKE, None, 4, 8, 128, 64, 16, 2, 1, 0) == -3    # f16 cache
    assert call(FAKE, FAKE, FAKE, FAKE, None, 4, 8, 128, 64, 16, 3, 4, 0) == -3    # fp8 source
    assert call(FAKE, FAKE, FAKE, FAKE, None, 4, 8, 120, 64, 16, 2, 4, 0) == -2    # D % 16
    assert call(FAKE, FAKE, FAKE, FAKE, None, 4, 8, 128, 64, 16, 2, 4, 3) == -2    # scale mode
    assert call(FAKE, FAKE, FAKE, None, None, 4, 8, 128, 64, 16, 2, 4, 0) == -1    # no scales
    assert call(None, None, None, None, None, 0, 8, 128, 64, 16, 2, 4, 0) == 0     # nothing to do


def test_append_status_codes():
    lib = pkv.load_library()
    call = lambda *a: lib.pkv_kv_append(*a, None)
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 64, 8, 1) == -2     # block size
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 64, 16, 3) == -3    # fp8
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 12, 64, 16, 1) == -2     # 24-byte rows
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 64, 16, 1) == -2
    assert call(None, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 64, 16, 1) == -1
    assert call(None, None, None, None, None, 0, 8, 128, 64, 16, 1) == 0     # nothing to do


@pytest.mark.parametrize("B,Hkv,maxb,parts", [
    (64, 8, 256, 1),        # 70B-shaped step
    (8, 8, 8192, 8),        # 131072-token fp8 case
    (64, 40, 100, 1),       # MHA prefix batch
    (4, 2, 7, 1),           # tiny
    (32, 8, 498, 2),        # Llama-3-8B layer
    (2, 2, 300, 19),        # few units: split down to 16-block partitions
])
def test_partition_plan(B, Hkv, maxb, parts):
    d = _dims(num_seqs=B, num_kv_heads=Hkv, num_q_heads=Hkv * 4, max_blocks_per_seq=maxb)
    assert pkv.decode_num_partitions(d) == parts
    ws = pkv.decode_workspace_bytes(d)
    assert ws == (0 if parts == 1 else B * Hkv * 4 * parts * (128 + 2) * 4)


def test_window_shrinks_the_partition_plan():
    # 16 sequences x 8 KV heads = 128 units -> 4 partitions of the full context
    d = _dims(num_seqs=16)
    assert pkv.decode_num_partitions(d) == 4
    # a 256-token window with 4 sinks attends at most 16 + 1 + 1 = 18 blocks
    d = _dims(num_seqs=16, window=256, sinks=4)
    assert pkv.decode_num_partitions(d) == 2          # 18 blocks, >= 16 per partition
    assert pkv.decode_workspace_bytes(d) == 16 * 64 * 2 * (128 + 2) * 4


def test_plan_uses_the_batch_size_hint_for_light_batches():
    # a table 8192 blocks wide, but the 8 sequences hold ~1000 blocks each:
    # sized for the width, 8 x 8 units would keep only 64 workgroups busy
    d = _dims(num_seqs=8, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=8192)
    assert pkv.decode_num_partitions(d) == 8                     # pieces of 1024
    d = _dims(num_seqs=8, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=8192, total_blocks=8000)
    assert pkv.decode_num_partitions(d) == -(-8192 // 125)       # pieces of 125
    # a batch that fills the chip keeps the default plan (Llama-3-8B-shaped)
    d = _dims(num_seqs=32, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=498, total_blocks=8704)
    assert pkv.decode_num_partitions(d) == 2
    # a uniform 70B-shaped batch is not split either way
    d = _dims(total_blocks=64 * 256)
    assert pkv.decode_num_partitions(d) == 1 and pkv.decode_workspace_bytes(d) == 0
    # a hint larger than the batch can hold is clamped to it
    d = _dims(num_seqs=8, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=8192, total_blocks=10 ** 9)
    assert pkv.decode_num_partitions(d) == 8
    assert _attn(_dims(total_blocks=-1)) == -2


def test_explicit_partition_size():
    d = _dims(partition_blocks=7)
    assert pkv.decode_num_partitions(d) == -(-256 // 7)
    d = _dims(partition_blocks=1000)
    assert pkv.decode_num_partitions(d) == 1 and pkv.decode_workspace_bytes(d) == 0


def test_status_strings():
    lib = pkv.load_library()
    for s in (0, -1, -2, -3, -4, -5, 9):
        assert lib.pkv_status_string(s)


def test_python_binding_rejects_host_tensors():
    q = torch.zeros(1, 4, 64)
    kc = torch.zeros(2, 1, 16, 64)
    with pytest.raises(ValueError):
        pkv.paged_decode_attn(q, kc, kc, torch.zeros(1, 2, dtype=torch.int32),
                              torch.ones(1, dtype=torch.int32), 0.125, torch.zeros_like(q))
    with pytest.raises(ValueError):
        pkv.kv_append(torch.zeros(1, 1, 64), torch.zeros(1, 1, 64), torch.zeros(1, dtype=torch.int64), kc, kc)


def test_noalloc_rejects_calls_beyond_its_scratch():
    """pkv_paged_decode_attn_noalloc: invalid arguments give the usual status,
    and a valid call whose split workspace would exceed the static scratch
    gives PKV_ERR_SCRATCH (-8) before anything touches the device."""
    lib = pkv.load_library()

    def call(dims, q=FAKE):
        return lib.pkv_paged_decode_attn_noalloc(q, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.088), FAKE,
                                                 ctypes.byref(dims), None)

    assert call(_dims(), q=None) == -1
    assert call(_dims(block_size=8)) == -2
    assert call(_dims(q_dtype=2)) == -3
    # 4096 sequences x 64 query heads x 16 pieces x (128 + 2) floats > 32 MiB
    big = _dims(num_seqs=4096, max_blocks_per_seq=256, partition_blocks=16)
    assert pkv.decode_workspace_bytes(big) > 32 * 2**20
    assert call(big) == -8
    assert lib.pkv_status_string(-8)


def test_k16_v8_and_per_token_status_codes():
    """A 16-bit K with an 8-bit V takes q and out of K's type, v_scales, and
    no K scales or channel factors; per-token flags are 0 or 1 and apply to
    an 8-bit K only.  All refused before any launch."""
    lib = pkv.load_library()

    def call(dims, v_dtype, ks=None, vs=FAKE, chan=None, k_tok=0, v_tok=0):
        qp = pkv.QuantParams(ks and ks.value, vs and vs.value, chan and chan.value, v_dtype, None, None,
                             None, 0, k_tok, v_tok)
        return lib.pkv_paged_decode_attn_quant(FAKE, FAKE, FAKE, ctypes.byref(qp), FAKE, FAKE,
                                               ctypes.c_float(0.088), FAKE, ctypes.byref(dims), None, 0,
                                               None)

    base = dict(num_q_heads=32, max_blocks_per_seq=16)
    f16 = _dims(**base, q_dtype=1, kv_dtype=1, out_dtype=1)
    bf16 = _dims(**base, q_dtype=2, kv_dtype=2, out_dtype=2)
    assert call(f16, 3, vs=None) == -1                       # V scales missing
    assert call(f16, 3, ks=FAKE) == -3                       # a 16-bit K takes no scales
    assert call(f16, 4, chan=FAKE) == -3                     # nor channel factors
    assert call(f16, 3, k_tok=1) == -3                       # nor per-token K scales
    assert call(bf16, 1) == -3                               # V must be 8-bit
    assert call(_dims(**base, q_dtype=2, kv_dtype=1, out_dtype=1), 3) == -3    # q of K's type
    assert call(_dims(**base, q_dtype=1, kv_dtype=1, out_dtype=0), 3) == -3    # out of K's type
    fp8 = _dims(**base, q_dtype=2, kv_dtype=3, out_dtype=2)
    assert call(fp8, 3, ks=FAKE, v_tok=2) == -2              # flags are 0 or 1
    assert call(fp8, 3, ks=FAKE, k_tok=-1) == -2
    assert call(fp8, 3, ks=None) == -1                       # an 8-bit K needs its scales


def test_quant_prefix_status_codes():
    """The group pass on 8-bit caches: K and V of one 8-bit format with
    per-(block, head) scales, q and out f16 or bf16 alike, head_dim 128; no
    channel factors, per-token scales or sink tiles.  All refused before
    any launch; a valid call asks for its workspace."""
    lib = pkv.load_library()

    def call(dims, v_dtype, ks=FAKE, vs=FAKE, chan=None, k_tok=0, v_tok=0, starts=FAKE, step=False):
        qp = pkv.QuantParams(ks and ks.value, vs and vs.value, chan and chan.value, v_dtype, None, None,
                             None, 0, k_tok, v_tok)
        if step:
            return lib.pkv_paged_decode_step_quant_prefix(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(qp),
                                                          starts, FAKE, FAKE, FAKE, ctypes.c_float(0.088),
                                                          FAKE, ctypes.byref(dims), None, 0, None)
        return lib.pkv_paged_decode_attn_quant_prefix(FAKE, FAKE, FAKE, ctypes.byref(qp), starts, FAKE, FAKE,
                                                      FAKE, ctypes.c_float(0.088), FAKE, ctypes.byref(dims),
                                                      None, 0, None)

    ok = dict(num_seqs=64, num_q_heads=40, num_kv_heads=40, max_blocks_per_seq=100, prefix_groups=1,
              prefix_max_seqs=64, prefix_max_blocks=75, kv_dtype=3, q_dtype=2, out_dtype=2)
    d = _dims(**ok)
    for step in (False, True):
        assert call(d, 3, step=step) == -4                          # valid, but no workspace
        assert call(d, 3, starts=None, step=step) == -1
        assert call(d, 3, ks=None, step=step) == -1
        assert call(d, 4, step=step) == -3                          # K fp8 with V int8
        assert call(d, 3, chan=FAKE, step=step) == -3
        assert call(d, 3, k_tok=1, step=step) == -3
        assert call(d, 3, v_tok=1, step=step) == -3
        assert call(_dims(**dict(ok, out_dtype=0)), 3, step=step) == -3        # out not q's type
        assert call(_dims(**dict(ok, q_dtype=0, out_dtype=0)), 3, step=step) == -3
        assert call(_dims(**dict(ok, head_dim=64)), 3, step=step) == -2
        assert call(_dims(**dict(ok, kv_dtype=1, q_dtype=1, out_dtype=1)), 3, step=step) == -3
    assert call(_dims(**dict(ok, kv_dtype=4)), 4) == -4             # int8 K and V: valid
    # the same plan and workspace as the 16-bit group pass
    assert pkv.decode_workspace_bytes(d) == 64 * 40 * (1 + 3) * (128 + 2) * 4


@pytest.mark.parametrize("kw,v_dtype,status", [
    (dict(head_dim=64), 1, -2),                        # the probe is for head_dim 128
    (dict(window=64), 1, -2),
    (dict(kv_dtype=0, q_dtype=0, out_dtype=0), 0, -3),  # f32 tiles
    (dict(kv_dtype=3), 1, -3),                         # V wider than K
    (dict(kv_dtype=1), 7, -3),                         # no such format
])
def test_paged_read_probe_status_codes(kw, v_dtype, status):
    lib = pkv.load_library()
    dims = _dims(**kw)
    assert lib.pkv_paged_read_probe(FAKE, FAKE, FAKE, FAKE, ctypes.byref(dims), v_dtype, FAKE, None) == status
    if status == -3:
        return
    dims = _dims()
    assert lib.pkv_paged_read_probe(None, FAKE, FAKE, FAKE, ctypes.byref(dims), 1, FAKE, None) == -1
