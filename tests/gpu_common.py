"""Helpers for the GPU parity tests: run the HIP step, feed the oracle.

The oracle always sees values that came from the seeded generator (copied to
the host before any HIP kernel ran on them) and applies its own append.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_56_amd as pkv

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2, "fp8_e4m3": 5e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_storage(t: torch.Tensor) -> np.ndarray:
    """Raw stored values as the oracle wants them (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def run_step(x, layer: int, spec, out: torch.Tensor, partition_blocks: int = 0,
             workspace=None, append: bool = True, window: int = 0, sinks: int = 0):
    """One layer of the decode step on the device: append, then attend."""
    kc, vc = x["k_cache"][layer], x["v_cache"][layer]
    kw = {}
    if spec.kv_dtype == "fp8_e4m3":
        kw = dict(k_scales=x["k_scales"][layer], v_scales=x["v_scales"][layer])
    if spec.append and append:
        if spec.kv_dtype == "fp8_e4m3":
            pkv.kv_append_fp8(x["k_new"][layer], x["v_new"][layer], x["slot_mapping"], kc, vc,
                              kw["k_scales"], kw["v_scales"])
        else:
            pkv.kv_append(x["k_new"][layer], x["v_new"][layer], x["slot_mapping"], kc, vc)
    return pkv.paged_decode_attn(x["q"][layer], kc, vc, x["block_tables"], x["context_lens"],
                                 spec.scale, out, workspace=workspace,
                                 partition_blocks=partition_blocks, window=window, sinks=sinks, **kw)


def oracle_rows(x_host_layer, layout, spec, seqs=None, q_heads=None, window=0, sinks=0):
    """Oracle output for the given rows from host copies of one layer's inputs.

    x_host_layer: dict with numpy storage arrays q, k_cache, v_cache (pre-append),
    k_new, v_new (if appending), k_scales, v_scales (fp8).
    """
    kc, vc, ks, vs = oracle_append(x_host_layer, spec, layout.slot_mapping)
    return oracle.paged_decode_attention(
        x_host_layer["q"], kc, vc, layout.block_tables, layout.context_lens, spec.scale,
        q_tag=spec.q_dtype, kv_tag=spec.kv_dtype, k_scales=ks, v_scales=vs,
        seqs=seqs, q_heads=q_heads, window=window, sinks=sinks)


def oracle_append(h, spec, slot_mapping):
    """The oracle's append for one layer's host copies: (k, v, k_scales, v_scales)."""
    kc, vc = h["k_cache"], h["v_cache"]
    ks, vs = h.get("k_scales"), h.get("v_scales")
    if spec.append:
        if spec.kv_dtype == "fp8_e4m3":
            kn = oracle.stored_to_f64(h["k_new"], spec.q_dtype).astype(np.float32)
            vn = oracle.stored_to_f64(h["v_new"], spec.q_dtype).astype(np.float32)
            kc, ks = oracle.kv_append_fp8(kc, ks, kn, slot_mapping, first_write=False)
            vc, vs = oracle.kv_append_fp8(vc, vs, vn, slot_mapping, first_write=False)
        else:
            kc = oracle.kv_append_bits(kc, h["k_new"], slot_mapping)
            vc = oracle.kv_append_bits(vc, h["v_new"], slot_mapping)
    return kc, vc, ks, vs


def host_layer(x, layer: int):
    h = {"q": host_storage(x["q"][layer]), "k_cache": host_storage(x["k_cache"][layer]),
         "v_cache": host_storage(x["v_cache"][layer])}
    for k in ("k_new", "v_new", "k_scales", "v_scales"):
        if k in x:
            h[k] = host_storage(x[k][layer])
    return h


def out_f64(out: torch.Tensor) -> np.ndarray:
    return out.detach().float().cpu().numpy().astype(np.float64)


def max_err(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0
