"""Workload descriptions (shapes, dtypes, length mixes, seeds).

Each workload is one decode step: every sequence appends the K/V of its new
token and then attends, with one query per head, over everything it has
cached.  Lengths are post-append lengths (the new token counts).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    seed: int
    num_layers: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str            # K's (and by default V's): "f32" | "f16" | "bf16" | "fp8_e4m3" | "int8"
    q_dtype: str             # "f32" | "f16" | "bf16"
    out_dtype: str           # "f32" | "f16" | "bf16"
    # Length mix: either explicit lengths, or uniform integers in [lo, hi].
    context_lens: Optional[Tuple[int, ...]] = None
    len_range: Optional[Tuple[int, int]] = None
    # Tokens shared by every sequence as a common prefix (whole blocks only).
    shared_prefix_tokens: int = 0
    # Physical pool size; None means exactly the blocks the batch needs.
    num_blocks: Optional[int] = None
    # Whether the step appends one new token per sequence before attending.
    append: bool = True
    block_size: int = 16
    description: str = ""
    # V's format when it differs from K's (8-bit caches only)
    v_dtype: Optional[str] = None
    # Outlier channels per KV head in K (x16); > 0 also gives K per-channel
    # factors equal to each channel's magnitude
    k_outliers: int = 0
    # 8-bit caches: the first this-many positions (<= 16) of every sequence
    # live in full-precision side tiles (q's dtype) instead of the cache
    fp_sinks: int = 0
    # 8-bit caches: one scale per (slot, KV head) instead of per (block, KV
    # head), for K and for V independently (per-token granularity)
    k_scale_tok: bool = False
    v_scale_tok: bool = False

    @property
    def v_tag(self) -> str:
        return self.v_dtype or self.kv_dtype

    @property
    def k_quantised(self) -> bool:
        return self.kv_dtype in ("fp8_e4m3", "int8")

    @property
    def quantised(self) -> bool:
        """Some cache is 8-bit (K, or V next to a 16-bit K)."""
        return self.k_quantised or self.v_tag in ("fp8_e4m3", "int8")

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5


WORKLOADS = {
    "tiny_f32": DecodeWorkload(
        name="tiny_f32", seed=56000, num_layers=1, num_seqs=4,
        num_q_heads=8, num_kv_heads=2, head_dim=64,
        kv_dtype="f32", q_dtype="f32", out_dtype="f32",
        context_lens=(17, 33, 64, 100), num_blocks=64, append=True,
        description="tiny fp32 decode, GQA-4, D=64, lens {17,33,64,100}, pool of 64 blocks",
    ),
    "llama3_8b_bf16": DecodeWorkload(
        name="llama3_8b_bf16", seed=56001, num_layers=1, num_seqs=32,
        num_q_heads=32, num_kv_heads=8, head_dim=128,
        kv_dtype="bf16", q_dtype="bf16", out_dtype="bf16",
        len_range=(512, 8192), append=True,
        description="Llama-3-8B-shaped layer, bf16, GQA-4, B=32, L~U[512,8192]",
    ),
    "llama70b_f16_80l": DecodeWorkload(
        name="llama70b_f16_80l", seed=56002, num_layers=80, num_seqs=64,
        num_q_heads=64, num_kv_heads=8, head_dim=128,
        kv_dtype="f16", q_dtype="f16", out_dtype="f16",
        context_lens=None, len_range=(4096, 4096), append=True,
        description="70B-shaped fp16 step, 80 layers, GQA-8, B=64 x 4096 tokens",
    ),
    "mha13b_prefix_f16": DecodeWorkload(
        name="mha13b_prefix_f16", seed=56003, num_layers=1, num_seqs=64,
        num_q_heads=40, num_kv_heads=40, head_dim=128,
        kv_dtype="f16", q_dtype="f16", out_dtype="f16",
        len_range=(50, 400), shared_prefix_tokens=1200, append=True,
        description="13B MHA fp16 layer, 64 seqs sharing a 1200-token prefix + U[50,400] suffix",
    ),
    "mha13b_prefix_bf16": DecodeWorkload(
        name="mha13b_prefix_bf16", seed=56010, num_layers=1, num_seqs=64,
        num_q_heads=40, num_kv_heads=40, head_dim=128,
        kv_dtype="bf16", q_dtype="bf16", out_dtype="bf16",
        len_range=(50, 400), shared_prefix_tokens=1200, append=True,
        description="13B MHA bf16 layer, 64 seqs sharing a 1200-token prefix + U[50,400] suffix",
    ),
    "mha13b_prefix_fp8": DecodeWorkload(
        name="mha13b_prefix_fp8", seed=56011, num_layers=1, num_seqs=64,
        num_q_heads=40, num_kv_heads=40, head_dim=128,
        kv_dtype="fp8_e4m3", q_dtype="bf16", out_dtype="bf16",
        len_range=(50, 400), shared_prefix_tokens=1200, append=True,
        description="13B MHA layer with an FP8 e4m3 cache, bf16 q/out, 64 seqs sharing a 1200-token "
                    "prefix + U[50,400] suffix",
    ),
    "long_fp8": DecodeWorkload(
        name="long_fp8", seed=56004, num_layers=1, num_seqs=8,
        num_q_heads=32, num_kv_heads=8, head_dim=128,
        kv_dtype="fp8_e4m3", q_dtype="bf16", out_dtype="bf16",
        len_range=(131072, 131072), append=True,
        description="long-context FP8 e4m3 KV, GQA-4, B=8 x 131072, bf16 q/out, split + merge",
    ),
    "long_fp8k_int8v": DecodeWorkload(
        name="long_fp8k_int8v", seed=56005, num_layers=1, num_seqs=8,
        num_q_heads=32, num_kv_heads=8, head_dim=128,
        kv_dtype="fp8_e4m3", v_dtype="int8", q_dtype="bf16", out_dtype="bf16",
        len_range=(131072, 131072), append=True,
        description="long-context mixed KV: K fp8 e4m3, V int8, GQA-4, B=8 x 131072, bf16 q/out",
    ),
    "long_int8_kchan": DecodeWorkload(
        name="long_int8_kchan", seed=56006, num_layers=1, num_seqs=8,
        num_q_heads=32, num_kv_heads=8, head_dim=128,
        kv_dtype="int8", q_dtype="bf16", out_dtype="bf16",
        len_range=(131072, 131072), append=True, k_outliers=4,
        description="long-context int8 KV, 4 outlier K channels per head with per-channel K "
                    "factors, GQA-4, B=8 x 131072, bf16 q/out",
    ),
    "long_bf16k_fp8v": DecodeWorkload(
        name="long_bf16k_fp8v", seed=56008, num_layers=1, num_seqs=8,
        num_q_heads=32, num_kv_heads=8, head_dim=128,
        kv_dtype="bf16", v_dtype="fp8_e4m3", q_dtype="bf16", out_dtype="bf16",
        len_range=(131072, 131072), append=True,
        description="long-context KV with V alone quantised: K bf16, V fp8 e4m3, GQA-4, "
                    "B=8 x 131072, bf16 q/out",
    ),
    "long_fp8_tok": DecodeWorkload(
        name="long_fp8_tok", seed=56009, num_layers=1, num_seqs=8,
        num_q_heads=32, num_kv_heads=8, head_dim=128,
        kv_dtype="fp8_e4m3", q_dtype="bf16", out_dtype="bf16",
        len_range=(131072, 131072), append=True, k_scale_tok=True, v_scale_tok=True,
        description="long-context FP8 e4m3 KV with one scale per (token, KV head), GQA-4, "
                    "B=8 x 131072, bf16 q/out",
    ),
    "llama70b_fp8_80l": DecodeWorkload(
        name="llama70b_fp8_80l", seed=56007, num_layers=80, num_seqs=64,
        num_q_heads=64, num_kv_heads=8, head_dim=128,
        kv_dtype="fp8_e4m3", q_dtype="f16", out_dtype="f16",
        context_lens=None, len_range=(4096, 4096), append=True,
        description="70B-shaped step with an FP8 e4m3 cache, 80 layers, GQA-8, B=64 x 4096 tokens, "
                    "f16 q/out",
    ),
}


def workload(name: str) -> DecodeWorkload:
    return WORKLOADS[name]


def scaled(w: DecodeWorkload, **changes) -> DecodeWorkload:
    """A copy of `w` with some fields replaced (smaller parity-test variants)."""
    return dataclasses.replace(w, **changes)
