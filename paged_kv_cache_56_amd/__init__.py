"""pagedkv: paged-KV decode attention for MI355X (gfx950), Python binding.

A thin ctypes layer over libpagedkv.so (include/pagedkv.h): it checks
tensor shapes and dtypes, passes raw device pointers and the current HIP
stream, and raises PagedKVError on a non-zero status.  All compute runs in
the library's HIP kernels; there is no fallback path.  torch tensors only
carry device memory and streams.

    kv_append(k_new, v_new, slot_mapping, k_cache, v_cache)
    kv_append_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scales, v_scales)
    kv_append_quant(x_new, slot_mapping, cache, scales, channel_scales=None)
    paged_decode_step(k_new, v_new, slot_mapping, q, k_cache, v_cache, block_tables,
                      context_lens, scale, out, workspace=None, partition_blocks=0,
                      window=0, sinks=0, total_blocks=0, prefix_group_starts=None,
                      prefix_group_blocks=None, prefix_max_seqs=0, prefix_max_blocks=0)
    paged_decode_attn(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                      k_scales=None, v_scales=None, k_channel_scales=None,
                      sink_k=None, sink_v=None, sink_tiles_of_seq=None,
                      workspace=None, partition_blocks=0, window=0, sinks=0,
                      total_blocks=0, prefix_group_starts=None, prefix_group_blocks=None,
                      prefix_max_seqs=0, prefix_max_blocks=0)
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PagedKVError",
    "library_path",
    "load_library",
    "kv_append",
    "kv_append_fp8",
    "kv_append_quant",
    "copy_blocks",
    "BlockManager",
    "paged_decode_attn",
    "paged_decode_step",
    "decode_dims",
    "decode_workspace_bytes",
    "decode_num_partitions",
    "hbm_read_probe",
    "paged_read_probe",
    "DTYPE_CODES",
    "BLOCK_SIZE",
]

BLOCK_SIZE = 16
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "lib", "libpagedkv.so")

DTYPE_CODES = {
    torch.float32: 0,
    torch.float16: 1,
    torch.bfloat16: 2,
    torch.uint8: 3,               # fp8 e4m3fn codes, stored as raw bytes
    torch.float8_e4m3fn: 3,
    torch.int8: 4,                # symmetric int8 codes
}
_Q8 = (3, 4)


class PagedKVError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"pagedkv status {status}: {msg}")
        self.status = status


class DecodeDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("partition_blocks", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("sinks", ctypes.c_int32),
        ("sink_tiles", ctypes.c_int32),
        ("total_blocks", ctypes.c_int32),
        ("prefix_groups", ctypes.c_int32),
        ("prefix_max_seqs", ctypes.c_int32),
        ("prefix_max_blocks", ctypes.c_int32),
    ]


class QuantParams(ctypes.Structure):
    _fields_ = [
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("k_channel_scales", ctypes.c_void_p),
        ("v_dtype", ctypes.c_int32),
        ("k_sink", ctypes.c_void_p),
        ("v_sink", ctypes.c_void_p),
        ("sink_tiles_of_seq", ctypes.c_void_p),
        ("num_sink_tiles", ctypes.c_int32),
        ("k_scales_per_token", ctypes.c_int32),
        ("v_scales_per_token", ctypes.c_int32),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libpagedkv.so (built in-tree by paged_kv_cache_56_amd._build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m paged_kv_cache_56_amd._build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    dims_p = ctypes.POINTER(DecodeDims)
    lib.pkv_kv_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.pkv_kv_append.restype = ctypes.c_int
    lib.pkv_kv_append_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.pkv_kv_append_fp8.restype = ctypes.c_int
    lib.pkv_kv_append_quant.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.pkv_kv_append_quant.restype = ctypes.c_int
    lib.pkv_decode_workspace_bytes.argtypes = [dims_p]
    lib.pkv_decode_workspace_bytes.restype = sz
    lib.pkv_decode_num_partitions.argtypes = [dims_p]
    lib.pkv_decode_num_partitions.restype = ctypes.c_int
    lib.pkv_paged_decode_attn.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, dims_p, vp, sz, vp]
    lib.pkv_paged_decode_attn.restype = ctypes.c_int
    lib.pkv_paged_decode_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, dims_p, vp]
    lib.pkv_paged_decode_attn_noalloc.restype = ctypes.c_int
    lib.pkv_paged_decode_attn_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                              dims_p, vp, sz, vp]
    lib.pkv_paged_decode_attn_fp8.restype = ctypes.c_int
    lib.pkv_paged_decode_attn_quant.argtypes = [vp, vp, vp, ctypes.POINTER(QuantParams), vp, vp,
                                                ctypes.c_float, vp, dims_p, vp, sz, vp]
    lib.pkv_paged_decode_attn_quant.restype = ctypes.c_int
    lib.pkv_paged_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, dims_p, vp,
                                          sz, vp]
    lib.pkv_paged_decode_step.restype = ctypes.c_int
    lib.pkv_paged_decode_step_quant.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(QuantParams), vp, vp,
                                                ctypes.c_float, vp, dims_p, vp, sz, vp]
    lib.pkv_paged_decode_step_quant.restype = ctypes.c_int
    lib.pkv_paged_decode_step_prefix.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                                 dims_p, vp, sz, vp]
    lib.pkv_paged_decode_step_prefix.restype = ctypes.c_int
    lib.pkv_paged_decode_attn_prefix.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                                 dims_p, vp, sz, vp]
    lib.pkv_paged_decode_attn_prefix.restype = ctypes.c_int
    lib.pkv_paged_decode_attn_quant_prefix.argtypes = [vp, vp, vp, ctypes.POINTER(QuantParams), vp, vp, vp, vp,
                                                       ctypes.c_float, vp, dims_p, vp, sz, vp]
    lib.pkv_paged_decode_attn_quant_prefix.restype = ctypes.c_int
    lib.pkv_paged_decode_step_quant_prefix.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(QuantParams), vp,
                                                       vp, vp, vp, ctypes.c_float, vp, dims_p, vp, sz, vp]
    lib.pkv_paged_decode_step_quant_prefix.restype = ctypes.c_int
    lib.pkv_paged_read_probe.argtypes = [vp, vp, vp, vp, dims_p, i32, vp, vp]
    lib.pkv_paged_read_probe.restype = ctypes.c_int
    lib.pkv_hbm_read_probe.argtypes = [vp, sz, vp, i32, vp]
    lib.pkv_hbm_read_probe.restype = ctypes.c_int
    i64, i32p, i64p = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    lib.pkv_copy_blocks.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.pkv_copy_blocks.restype = ctypes.c_int
    lib.pkv_bm_create.argtypes = [i32, i32, i32p]
    lib.pkv_bm_create.restype = vp
    lib.pkv_bm_destroy.argtypes = [vp]
    lib.pkv_bm_destroy.restype = None
    lib.pkv_bm_add_sequence.argtypes = [vp, i64]
    lib.pkv_bm_fork.argtypes = [vp, i64, i64]
    lib.pkv_bm_append_slots.argtypes = [vp, i64p, i32, i64p, i32p, i32p, i32, i32p]
    lib.pkv_bm_free_sequence.argtypes = [vp, i64]
    lib.pkv_bm_num_free.argtypes = [vp]
    lib.pkv_bm_refcount.argtypes = [vp, i32]
    lib.pkv_bm_block_tables.argtypes = [vp, i64p, i32, i32, i32p, i32p]
    for f in ("pkv_bm_add_sequence", "pkv_bm_fork", "pkv_bm_append_slots", "pkv_bm_free_sequence",
              "pkv_bm_num_free", "pkv_bm_refcount", "pkv_bm_block_tables"):
        getattr(lib, f).restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().pkv_status_string(status).decode()
        raise PagedKVError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev(*ts) -> None:
    dev = None
    for t in ts:
        if t is None:
            continue
        _need(t.is_cuda, "all tensors must be on the GPU")
        _need(t.is_contiguous(), "all tensors must be contiguous")
        dev = dev or t.device
        _need(t.device == dev, "all tensors must be on one device")


def _code(t: torch.Tensor) -> int:
    if t.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return DTYPE_CODES[t.dtype]


def kv_append(k_new: torch.Tensor, v_new: Optional[torch.Tensor], slot_mapping: torch.Tensor,
              k_cache: torch.Tensor, v_cache: Optional[torch.Tensor]) -> None:
    """Write token t's K/V rows into slot slot_mapping[t] (-1 = skip).

    k_new, v_new: [T, Hkv, D]; slot_mapping: int64 [T];
    caches: [num_blocks, Hkv, 16, D] of the same dtype.  v_new and v_cache
    both None: K alone (a 16-bit K next to an 8-bit V).
    """
    lib = load_library()
    _dev(k_new, v_new, slot_mapping, k_cache, v_cache)
    _need((v_new is None) == (v_cache is None), "v_new and v_cache go together")
    _need(k_new.dim() == 3 and (v_new is None or k_new.shape == v_new.shape), "k_new/v_new must be [T, Hkv, D]")
    _need(k_cache.dim() == 4 and (v_cache is None or k_cache.shape == v_cache.shape),
          "caches must be [NB, Hkv, 16, D]")
    T, H, D = k_new.shape
    _need(k_cache.shape[1] == H and k_cache.shape[3] == D, "cache and new-token shapes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (T,), "slot_mapping must be int64 [T]")
    _need(k_new.dtype == k_cache.dtype and (v_new is None or v_new.dtype == v_cache.dtype == k_cache.dtype),
          "dtype mismatch")
    _check(lib.pkv_kv_append(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache),
                             _ptr(v_cache), T, H, D, k_cache.shape[0], k_cache.shape[2],
                             _code(k_cache), _stream(k_cache)))


SCALE_GIVEN, SCALE_FIRST_WRITE, SCALE_PER_TOKEN = 0, 1, 2


def kv_append_fp8(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor, k_scales: torch.Tensor,
                  v_scales: torch.Tensor, *, first_write: bool = False) -> None:
    """Quantise token t's K/V rows (f32/f16/bf16) into fp8 e4m3 caches at its slot.

    k_new, v_new: [T, Hkv, D]; caches: uint8 or float8_e4m3fn [NB, Hkv, 16, D];
    scales: fp32 [NB, Hkv].  With first_write=True the token that opens a block
    sets that block's scale to max|x|/448 first; otherwise the given scales are used.
    """
    lib = load_library()
    _dev(k_new, v_new, slot_mapping, k_cache, v_cache, k_scales, v_scales)
    _need(k_new.shape == v_new.shape and k_new.dim() == 3, "k_new/v_new must be [T, Hkv, D]")
    _need(k_cache.shape == v_cache.shape and k_cache.dim() == 4 and _code(k_cache) == 3,
          "caches must be fp8 [NB, Hkv, 16, D]")
    T, H, D = k_new.shape
    _need(k_cache.shape[1] == H and k_cache.shape[3] == D, "cache and new-token shapes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (T,), "slot_mapping must be int64 [T]")
    _need(k_scales.dtype == v_scales.dtype == torch.float32 and
          k_scales.shape == v_scales.shape == k_cache.shape[:2], "scales must be fp32 [NB, Hkv]")
    _need(k_new.dtype == v_new.dtype and _code(k_new) in (0, 1, 2), "k_new/v_new must be f32/f16/bf16")
    _check(lib.pkv_kv_append_fp8(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), T, H, D,
                                 k_cache.shape[0], k_cache.shape[2], _code(k_new),
                                 SCALE_FIRST_WRITE if first_write else SCALE_GIVEN, _stream(k_cache)))


def kv_append_quant(x_new: torch.Tensor, slot_mapping: torch.Tensor, cache: torch.Tensor,
                    scales: torch.Tensor, *, channel_scales: Optional[torch.Tensor] = None,
                    first_write: bool = False) -> None:
    """Quantise token t's rows (f32/f16/bf16) into ONE 8-bit cache at its slot.

    x_new: [T, Hkv, D]; cache: fp8 (uint8 / float8_e4m3fn) or int8 [NB, Hkv, 16, D];
    scales: fp32 [NB, Hkv], or fp32 [NB, Hkv, 16] for one scale per (slot, head)
    (every token then sets its own from its row); channel_scales: optional fp32
    [Hkv, D] that each element is divided by first.  first_write as in
    kv_append_fp8 (QMAX 448 for fp8, 127 for int8).
    """
    lib = load_library()
    _dev(x_new, slot_mapping, cache, scales, channel_scales)
    _need(x_new.dim() == 3 and cache.dim() == 4 and _code(cache) in _Q8,
          "x_new must be [T, Hkv, D] and the cache 8-bit [NB, Hkv, 16, D]")
    T, H, D = x_new.shape
    _need(cache.shape[1] == H and cache.shape[3] == D, "cache and new-token shapes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (T,), "slot_mapping must be int64 [T]")
    per_token = scales.dim() == 3
    _need(scales.dtype == torch.float32 and scales.shape in (cache.shape[:2], cache.shape[:3]),
          "scales must be fp32 [NB, Hkv] or [NB, Hkv, 16]")
    _need(not (per_token and first_write), "per-token scales are always set by their token")
    _need(channel_scales is None or (channel_scales.dtype == torch.float32 and
                                     channel_scales.shape == (H, D)), "channel_scales must be fp32 [Hkv, D]")
    _need(_code(x_new) in (0, 1, 2), "x_new must be f32/f16/bf16")
    _check(lib.pkv_kv_append_quant(_ptr(x_new), _ptr(slot_mapping), _ptr(cache), _ptr(scales),
                                   _ptr(channel_scales), T, H, D, cache.shape[0], cache.shape[2],
                                   _code(x_new), _code(cache),
                                   SCALE_PER_TOKEN if per_token else
                                   (SCALE_FIRST_WRITE if first_write else SCALE_GIVEN), _stream(cache)))


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src: torch.Tensor, dst: torch.Tensor,
                k_scales: Optional[torch.Tensor] = None, v_scales: Optional[torch.Tensor] = None) -> None:
    """Copy-on-write: blocks dst[i] of both caches (and 8-bit scales) become bit
    copies of blocks src[i].  src, dst: int32 [n] on the device."""
    lib = load_library()
    _dev(k_cache, v_cache, src, dst, k_scales, v_scales)
    _need(k_cache.shape == v_cache.shape and k_cache.dim() == 4, "caches must be [NB, Hkv, 16, D]")
    _need(k_cache.element_size() == v_cache.element_size(), "K and V elements differ in width")
    _need(src.dtype == dst.dtype == torch.int32 and src.shape == dst.shape and src.dim() == 1,
          "src/dst must be int32 [n]")
    NB, H, _, D = k_cache.shape
    _check(lib.pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _ptr(src),
                               _ptr(dst), src.numel(), H, D, NB, _code(k_cache), _stream(k_cache)))


class BlockManager:
    """The library's host block manager (pool, reference counts, fork,
    copy-on-write).  See pkv_bm_* in include/pagedkv.h."""

    def __init__(self, num_blocks: int, free_order=None, block_size: int = BLOCK_SIZE):
        self._lib = load_library()
        order = None
        if free_order is not None:
            arr = (ctypes.c_int32 * num_blocks)(*[int(b) for b in free_order])
            order = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
        self._h = self._lib.pkv_bm_create(num_blocks, block_size, order)
        if not self._h:
            raise ValueError("bad block manager arguments")
        self.num_blocks = num_blocks

    def close(self) -> None:
        if self._h:
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self, seq: int) -> None:
        _check(self._lib.pkv_bm_add_sequence(self._h, seq))

    def fork(self, parent: int, child: int) -> None:
        _check(self._lib.pkv_bm_fork(self._h, parent, child))

    def append_slots(self, seqs):
        """-> (slots list, [(src_block, dst_block), ...] to copy first)."""
        n = len(seqs)
        sq = (ctypes.c_int64 * max(n, 1))(*seqs)
        slots = (ctypes.c_int64 * max(n, 1))()
        cs = (ctypes.c_int32 * max(n, 1))()
        cd = (ctypes.c_int32 * max(n, 1))()
        nc = ctypes.c_int32(0)
        _check(self._lib.pkv_bm_append_slots(self._h, sq, n, slots, cs, cd, max(n, 1), ctypes.byref(nc)))
        return list(slots[:n]), [(cs[i], cd[i]) for i in range(nc.value)]

    def free_sequence(self, seq: int) -> None:
        _check(self._lib.pkv_bm_free_sequence(self._h, seq))

    def num_free(self) -> int:
        n = self._lib.pkv_bm_num_free(self._h)
        _check(min(n, 0))
        return n

    def refcount(self, block: int) -> int:
        n = self._lib.pkv_bm_refcount(self._h, block)
        _check(min(n, 0))
        return n

    def block_tables(self, seqs, max_blocks: int):
        """-> (int32 tensor [n, max_blocks] padded with -1, int32 tensor [n] lengths), on the CPU."""
        n = len(seqs)
        tables = torch.empty((max(n, 1), max_blocks), dtype=torch.int32)
        lens = torch.empty((max(n, 1),), dtype=torch.int32)
        sq = (ctypes.c_int64 * max(n, 1))(*seqs)
        _check(self._lib.pkv_bm_block_tables(
            self._h, sq, n, max_blocks, ctypes.cast(tables.data_ptr(), ctypes.POINTER(ctypes.c_int32)),
            ctypes.cast(lens.data_ptr(), ctypes.POINTER(ctypes.c_int32))))
        return tables[:n], lens[:n]


def decode_dims(q: torch.Tensor, k_cache: torch.Tensor, block_tables: torch.Tensor,
                out: torch.Tensor, partition_blocks: int = 0, window: int = 0,
                sinks: int = 0, sink_tiles: bool = False, total_blocks: int = 0,
                prefix_groups: int = 0, prefix_max_seqs: int = 0,
                prefix_max_blocks: int = 0) -> DecodeDims:
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    _need(Dk == D, "head_dim of q and cache differ")
    return DecodeDims(B, Hq, Hkv, D, bs, NB, block_tables.shape[1], _code(q), _code(k_cache),
                      _code(out), partition_blocks, window, sinks, int(sink_tiles), int(total_blocks),
                      int(prefix_groups), int(prefix_max_seqs), int(prefix_max_blocks))


def decode_workspace_bytes(dims: DecodeDims) -> int:
    return int(load_library().pkv_decode_workspace_bytes(ctypes.byref(dims)))


def decode_num_partitions(dims: DecodeDims) -> int:
    n = load_library().pkv_decode_num_partitions(ctypes.byref(dims))
    _check(min(n, 0))
    return n


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Read every byte of `buf` once (bandwidth reference); sink: int32 [W] on the device."""
    _dev(buf, sink)
    _need(sink.dtype == torch.int32 and sink.dim() == 1, "sink must be int32 [workgroups]")
    _check(load_library().pkv_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                             sink.numel(), _stream(buf)))


def paged_read_probe(k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                     context_lens: torch.Tensor, dims: DecodeDims, sink: torch.Tensor) -> None:
    """The attention call's memory traffic for `dims` without its arithmetic
    (bandwidth reference); sink: int32 [B * Hkv * partitions] on the device.
    dims.kv_dtype is K's format; V's is taken from v_cache's dtype (a 16-bit
    K may go with an 8-bit V)."""
    _dev(k_cache, v_cache, block_tables, context_lens, sink)
    _need(sink.dtype == torch.int32 and sink.dim() == 1 and
          sink.numel() >= dims.num_seqs * dims.num_kv_heads * decode_num_partitions(dims),
          "sink must be int32 [B * Hkv * partitions]")
    _check(load_library().pkv_paged_read_probe(_ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                               _ptr(context_lens), ctypes.byref(dims), _code(v_cache),
                                               _ptr(sink), _stream(k_cache)))


def paged_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      out: torch.Tensor, *, k_scales: Optional[torch.Tensor] = None,
                      v_scales: Optional[torch.Tensor] = None,
                      k_channel_scales: Optional[torch.Tensor] = None,
                      sink_k: Optional[torch.Tensor] = None, sink_v: Optional[torch.Tensor] = None,
                      sink_tiles_of_seq: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      partition_blocks: int = 0, window: int = 0, sinks: int = 0,
                      total_blocks: int = 0,
                      prefix_group_starts: Optional[torch.Tensor] = None,
                      prefix_group_blocks: Optional[torch.Tensor] = None,
                      prefix_max_seqs: int = 0, prefix_max_blocks: int = 0) -> torch.Tensor:
    """out[b, i] = softmax(scale * q[b, i] . K^T) V over the first context_lens[b]
    tokens of sequence b, K/V read through block_tables.  Returns `out`.

    q, out: [B, Hq, D]; caches: [NB, Hkv, 16, D]; block_tables: int32 [B, max_blocks];
    context_lens: int32 [B].  8-bit caches -- fp8 (uint8 or float8_e4m3fn) or
    int8, K fp8 with V int8 allowed, or a 16-bit K (q's dtype) with an 8-bit V --
    need k_scales (8-bit K only) and v_scales: fp32 [NB, Hkv], or [NB, Hkv, 16]
    for one scale per (slot, head); an 8-bit K may give k_channel_scales: fp32
    [Hkv, D], and the caller may give full-precision sink
    tiles sink_k, sink_v: [num_tiles, Hkv, 16, D] of q's dtype with
    sink_tiles_of_seq: int32 [B] (positions < sinks of sequence b are read from
    its tile; 1 <= sinks <= 16, with or without a window).  total_blocks (the
    batch's sum of ceil(len / 16), known to a scheduler on the host) lets the
    split plan balance uneven lengths.  `workspace` (uint8, on the device) is allocated here
    when the call splits the context and none is given.  window > 0 limits each
    query to the last `window` positions plus the first `sinks` positions.

    Shared prefixes: prefix_group_starts int32 [G + 1] (nondecreasing; group g
    = sequences [starts[g], starts[g + 1])) and prefix_group_blocks int32 [G]
    (the group's shared leading table entries, full blocks) on the device,
    with host bounds prefix_max_seqs (>= every group's size) and
    prefix_max_blocks (>= every count); the shared blocks are then read once
    per group.  The result is the same attention.  Caches f16 or bf16 with q
    and out alike, or K and V of one 8-bit format with per-(block, head)
    scales, q and out f16 or bf16, head_dim 128 (no channel factors,
    per-token scales or sink tiles).
    """
    lib = load_library()
    _dev(q, k_cache, v_cache, block_tables, context_lens, out, k_scales, v_scales, k_channel_scales,
         sink_k, sink_v, sink_tiles_of_seq, workspace, prefix_group_starts, prefix_group_blocks)
    _need(q.dim() == 3 and out.shape == q.shape, "q and out must be [B, Hq, D]")
    _need(k_cache.shape == v_cache.shape and k_cache.dim() == 4, "caches must be [NB, Hkv, 16, D]")
    kc, vc = _code(k_cache), _code(v_cache)
    _need(kc == vc or (vc in _Q8 and (kc in _Q8 or kc in (1, 2))),
          "K and V caches differ in dtype (an 8-bit V may go with an 8-bit or a 16-bit K)")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == q.shape[0], "block_tables must be int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
          "context_lens must be int32 [B]")
    side = sink_k is not None or sink_v is not None or sink_tiles_of_seq is not None
    if side:
        _need(sink_k is not None and sink_v is not None and sink_tiles_of_seq is not None,
              "full-precision sinks need sink_k, sink_v and sink_tiles_of_seq")
        _need(sink_k.shape == sink_v.shape and sink_k.dim() == 4 and sink_k.shape[1:] == k_cache.shape[1:]
              and sink_k.dtype == sink_v.dtype == q.dtype, "sink tiles must be [n, Hkv, 16, D] of q's dtype")
        _need(sink_tiles_of_seq.dtype == torch.int32 and sink_tiles_of_seq.shape == (q.shape[0],),
              "sink_tiles_of_seq must be int32 [B]")
    grouped = prefix_group_starts is not None or prefix_group_blocks is not None
    G = 0
    if grouped:
        _need(prefix_group_starts is not None and prefix_group_blocks is not None,
              "shared prefixes need prefix_group_starts and prefix_group_blocks")
        G = prefix_group_blocks.numel()
        _need(prefix_group_starts.dtype == prefix_group_blocks.dtype == torch.int32
              and prefix_group_blocks.dim() == 1 and prefix_group_starts.shape == (G + 1,),
              "prefix_group_starts must be int32 [G + 1] and prefix_group_blocks int32 [G]")
        _need(kc == vc and (kc in (1, 2) or kc in _Q8),
              "shared prefixes need f16 or bf16 caches, or K and V of one 8-bit format")
    dims = decode_dims(q, k_cache, block_tables, out, partition_blocks, window, sinks, side, total_blocks,
                       G, prefix_max_seqs if grouped else 0, prefix_max_blocks if grouped else 0)
    need = decode_workspace_bytes(dims)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if (need and workspace is not None) else 0
    if vc in _Q8:
        k8 = kc in _Q8
        _need(v_scales is not None and (k_scales is not None) == k8,
              "an 8-bit V needs v_scales, an 8-bit K k_scales (a 16-bit K takes none)")
        for sc in (k_scales, v_scales):
            _need(sc is None or (sc.dtype == torch.float32 and
                                 sc.shape in (k_cache.shape[:2], k_cache.shape[:3])),
                  "scales must be fp32 [NB, Hkv], or [NB, Hkv, 16] for one per (slot, head)")
        k_tok = int(k_scales is not None and k_scales.dim() == 3)
        v_tok = int(v_scales.dim() == 3)
        _need(k_channel_scales is None or (k8 and k_channel_scales.dtype == torch.float32 and
                                           k_channel_scales.shape == (k_cache.shape[1], k_cache.shape[3])),
              "k_channel_scales must be fp32 [Hkv, D], for an 8-bit K")
        if grouped:
            qp = QuantParams(_ptr(k_scales), _ptr(v_scales), _ptr(k_channel_scales), vc,
                             None, None, None, 0, k_tok, v_tok)
            st = lib.pkv_paged_decode_attn_quant_prefix(_ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(qp),
                                                        _ptr(prefix_group_starts), _ptr(prefix_group_blocks),
                                                        _ptr(block_tables), _ptr(context_lens), float(scale),
                                                        _ptr(out), ctypes.byref(dims), ws_ptr, ws_bytes,
                                                        _stream(q))
        elif kc == vc == 3 and k_channel_scales is None and not side and not (k_tok or v_tok):
            st = lib.pkv_paged_decode_attn_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales),
                                               _ptr(v_scales), _ptr(block_tables), _ptr(context_lens),
                                               float(scale), _ptr(out), ctypes.byref(dims), ws_ptr,
                                               ws_bytes, _stream(q))
        else:
            qp = QuantParams(_ptr(k_scales), _ptr(v_scales), _ptr(k_channel_scales), vc,
                             _ptr(sink_k), _ptr(sink_v), _ptr(sink_tiles_of_seq),
                             sink_k.shape[0] if side else 0, k_tok, v_tok)
            st = lib.pkv_paged_decode_attn_quant(_ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(qp),
                                                 _ptr(block_tables), _ptr(context_lens), float(scale),
                                                 _ptr(out), ctypes.byref(dims), ws_ptr, ws_bytes,
                                                 _stream(q))
    else:
        _need(k_scales is None and v_scales is None and k_channel_scales is None and not side,
              "scales and sink tiles apply to 8-bit caches only")
        if grouped:
            st = lib.pkv_paged_decode_attn_prefix(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                  _ptr(prefix_group_starts), _ptr(prefix_group_blocks),
                                                  _ptr(block_tables), _ptr(context_lens), float(scale),
                                                  _ptr(out), ctypes.byref(dims), ws_ptr, ws_bytes,
                                                  _stream(q))
        else:
            st = lib.pkv_paged_decode_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                           _ptr(context_lens), float(scale), _ptr(out),
                                           ctypes.byref(dims), ws_ptr, ws_bytes, _stream(q))
    _check(st)
    return out


def paged_decode_step(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                      q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      out: torch.Tensor, *, workspace: Optional[torch.Tensor] = None,
                      partition_blocks: int = 0, window: int = 0, sinks: int = 0,
                      total_blocks: int = 0,
                      prefix_group_starts: Optional[torch.Tensor] = None,
                      prefix_group_blocks: Optional[torch.Tensor] = None,
                      prefix_max_seqs: int = 0, prefix_max_blocks: int = 0,
                      k_scales: Optional[torch.Tensor] = None, v_scales: Optional[torch.Tensor] = None,
                      k_channel_scales: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kv_append of each sequence's new token, then paged_decode_attn, in one launch.

    k_new, v_new: [B, Hkv, D] (row b is sequence b's new token); slot_mapping:
    int64 [B], the slot of sequence b's last position (-1: none).  Caches and
    q/out f32, f16 or bf16 of one type.  Shared-prefix groups (f16/bf16) as in
    paged_decode_attn; each new token must then lie past its group's shared
    blocks.  8-bit caches (as in paged_decode_attn, no sink tiles): k_new and
    v_new in q's dtype, quantised on write with the blocks' given scales, or
    setting their own slot's scale when the scales are per token; with
    shared-prefix groups, the limits paged_decode_attn states for them.
    Returns `out`.
    """
    lib = load_library()
    _dev(k_new, v_new, slot_mapping, q, k_cache, v_cache, block_tables, context_lens, out, workspace,
         prefix_group_starts, prefix_group_blocks, k_scales, v_scales, k_channel_scales)
    _need(q.dim() == 3 and out.shape == q.shape, "q and out must be [B, Hq, D]")
    _need(k_cache.shape == v_cache.shape and k_cache.dim() == 4, "caches must be [NB, Hkv, 16, D]")
    B = q.shape[0]
    _need(k_new.shape == v_new.shape == (B, k_cache.shape[1], k_cache.shape[3]),
          "k_new/v_new must be [B, Hkv, D]")
    kc, vc = _code(k_cache), _code(v_cache)
    grouped = prefix_group_starts is not None or prefix_group_blocks is not None
    G = 0
    if grouped:
        _need(prefix_group_starts is not None and prefix_group_blocks is not None,
              "shared prefixes need prefix_group_starts and prefix_group_blocks")
        G = prefix_group_blocks.numel()
        _need(prefix_group_starts.dtype == prefix_group_blocks.dtype == torch.int32
              and prefix_group_blocks.dim() == 1 and prefix_group_starts.shape == (G + 1,),
              "prefix_group_starts must be int32 [G + 1] and prefix_group_blocks int32 [G]")
    if vc in _Q8:
        _need(k_new.dtype == v_new.dtype == q.dtype, "new rows of an 8-bit cache come in q's dtype")
        _need(not grouped or kc == vc, "shared prefixes need K and V of one 8-bit format")
        k8 = kc in _Q8
        _need(kc in _Q8 or kc == _code(q), "K and V caches differ in dtype")
        _need(v_scales is not None and (k_scales is not None) == k8,
              "an 8-bit V needs v_scales, an 8-bit K k_scales (a 16-bit K takes none)")
        for sc in (k_scales, v_scales):
            _need(sc is None or (sc.dtype == torch.float32 and
                                 sc.shape in (k_cache.shape[:2], k_cache.shape[:3])),
                  "scales must be fp32 [NB, Hkv], or [NB, Hkv, 16] for one per (slot, head)")
        _need(k_channel_scales is None or (k8 and k_channel_scales.dtype == torch.float32 and
                                           k_channel_scales.shape == (k_cache.shape[1], k_cache.shape[3])),
              "k_channel_scales must be fp32 [Hkv, D], for an 8-bit K")
        dims = decode_dims(q, k_cache, block_tables, out, partition_blocks, window, sinks, False, total_blocks,
                           G, prefix_max_seqs if grouped else 0, prefix_max_blocks if grouped else 0)
        need = decode_workspace_bytes(dims)
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        qp = QuantParams(_ptr(k_scales), _ptr(v_scales), _ptr(k_channel_scales), vc, None, None, None, 0,
                         int(k_scales is not None and k_scales.dim() == 3), int(v_scales.dim() == 3))
        ws_ptr = _ptr(workspace) if need else None
        ws_bytes = workspace.numel() * workspace.element_size() if need else 0
        if grouped:
            st = lib.pkv_paged_decode_step_quant_prefix(
                _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                ctypes.byref(qp), _ptr(prefix_group_starts), _ptr(prefix_group_blocks), _ptr(block_tables),
                _ptr(context_lens), float(scale), _ptr(out), ctypes.byref(dims), ws_ptr, ws_bytes, _stream(q))
        else:
            st = lib.pkv_paged_decode_step_quant(
                _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                ctypes.byref(qp), _ptr(block_tables), _ptr(context_lens), float(scale), _ptr(out),
                ctypes.byref(dims), ws_ptr, ws_bytes, _stream(q))
        _check(st)
        return out
    _need(k_scales is None and v_scales is None and k_channel_scales is None,
          "scales apply to 8-bit caches only")
    _need(k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype, "dtype mismatch")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (B,), "slot_mapping must be int64 [B]")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
          "block_tables must be int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (B,), "context_lens must be int32 [B]")
    dims = decode_dims(q, k_cache, block_tables, out, partition_blocks, window, sinks, False, total_blocks,
                       G, prefix_max_seqs if grouped else 0, prefix_max_blocks if grouped else 0)
    need = decode_workspace_bytes(dims)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if (need and workspace is not None) else 0
    if grouped:
        st = lib.pkv_paged_decode_step_prefix(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(q),
                                              _ptr(k_cache), _ptr(v_cache), _ptr(prefix_group_starts),
                                              _ptr(prefix_group_blocks), _ptr(block_tables),
                                              _ptr(context_lens), float(scale), _ptr(out),
                                              ctypes.byref(dims), ws_ptr, ws_bytes, _stream(q))
    else:
        st = lib.pkv_paged_decode_step(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(q), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), float(scale),
                                       _ptr(out), ctypes.byref(dims), ws_ptr, ws_bytes, _stream(q))
    _check(st)
    return out
