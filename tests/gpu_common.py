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

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2, "fp8_e4m3": 5e-2, "int8": 5e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_storage(t: torch.Tensor) -> np.ndarray:
    """Raw stored values as the oracle wants them (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.int8:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def group_args(x) -> dict:
    """Shared-prefix group arguments of the attention call, from the tensors'
    group descriptors (host bounds as a scheduler would know them)."""
    starts, blocks = x["group_starts"], x["group_blocks"]
    hs = starts.cpu().numpy()
    return dict(prefix_group_starts=starts, prefix_group_blocks=blocks,
                prefix_max_seqs=max(1, int((hs[1:] - hs[:-1]).max(initial=0))),
                prefix_max_blocks=int(blocks.cpu().numpy().max(initial=0)))


def run_step(x, layer: int, spec, out: torch.Tensor, partition_blocks: int = 0,
             workspace=None, append: bool = True, window: int = 0, sinks: int = 0,
             balanced: bool = False, grouped: bool = False):
    """One layer of the decode step on the device: append, then attend.
    balanced: pass the batch's block count, as a scheduler would.
    grouped: read shared prefixes once per group (the tensors' descriptors)."""
    total_blocks = int(((x["context_lens"].cpu().long() + 15) // 16).sum()) if balanced else 0
    kc, vc = x["k_cache"][layer], x["v_cache"][layer]
    kw = {}
    chan = x.get("k_channel_scales")
    if spec.quantised:
        kw = dict(v_scales=x["v_scales"][layer])
        if spec.k_quantised:
            kw["k_scales"] = x["k_scales"][layer]
        if chan is not None:
            kw["k_channel_scales"] = chan
    if spec.fp_sinks:
        kw.update(sink_k=x["sink_k"][layer], sink_v=x["sink_v"][layer],
                  sink_tiles_of_seq=x["sink_tiles_of_seq"])
        sinks = spec.fp_sinks
        if spec.append and append:      # a new token among the first S goes to its tile
            pkv.kv_append(x["k_new"][layer], x["v_new"][layer], x["sink_slot_mapping"],
                          x["sink_k"][layer], x["sink_v"][layer])
    if spec.append and append:
        if (spec.kv_dtype == spec.v_tag == "fp8_e4m3" and chan is None
                and not (spec.k_scale_tok or spec.v_scale_tok)):
            pkv.kv_append_fp8(x["k_new"][layer], x["v_new"][layer], x["slot_mapping"], kc, vc,
                              kw["k_scales"], kw["v_scales"])
        elif spec.quantised:
            if spec.k_quantised:
                pkv.kv_append_quant(x["k_new"][layer], x["slot_mapping"], kc, kw["k_scales"],
                                    channel_scales=chan)
            else:                                   # a 16-bit K: a bit copy of K alone
                pkv.kv_append(x["k_new"][layer], None, x["slot_mapping"], kc, None)
            pkv.kv_append_quant(x["v_new"][layer], x["slot_mapping"], vc, kw["v_scales"])
        else:
            pkv.kv_append(x["k_new"][layer], x["v_new"][layer], x["slot_mapping"], kc, vc)
    if grouped:
        kw.update(group_args(x))
    return pkv.paged_decode_attn(x["q"][layer], kc, vc, x["block_tables"], x["context_lens"],
                                 spec.scale, out, workspace=workspace,
                                 partition_blocks=partition_blocks, window=window, sinks=sinks,
                                 total_blocks=total_blocks, **kw)


def oracle_rows(x_host_layer, layout, spec, seqs=None, q_heads=None, window=0, sinks=0):
    """Oracle output for the given rows from host copies of one layer's inputs.

    x_host_layer: dict with numpy storage arrays q, k_cache, v_cache (pre-append),
    k_new, v_new (if appending), k_scales, v_scales (8-bit), k_channel_scales.
    """
    kc, vc, ks, vs = oracle_append(x_host_layer, spec, layout.slot_mapping)
    return oracle_attend(x_host_layer, spec, kc, vc, ks, vs, layout.block_tables, layout.context_lens,
                         seqs=seqs, q_heads=q_heads, window=window, sinks=sinks)


def oracle_attend(h, spec, kc, vc, ks, vs, tables, lens, seqs=None, q_heads=None, window=0, sinks=0):
    """The oracle's attention on one layer's (appended) host copies."""
    side = {}
    if spec.fp_sinks:
        sk, sv = h["sink_k"], h["sink_v"]
        if spec.append:
            sk = oracle.kv_append_bits(sk, h["k_new"], h["sink_slot_mapping"])
            sv = oracle.kv_append_bits(sv, h["v_new"], h["sink_slot_mapping"])
        side = dict(sink_k=sk, sink_v=sv, sink_blocks=h["sink_tiles_of_seq"])
        sinks = spec.fp_sinks
    return oracle.paged_decode_attention(
        h["q"], kc, vc, tables, lens, spec.scale,
        q_tag=spec.q_dtype, kv_tag=spec.kv_dtype, v_tag=spec.v_tag, k_scales=ks, v_scales=vs,
        k_channel_scales=h.get("k_channel_scales"),
        seqs=seqs, q_heads=q_heads, window=window, sinks=sinks, **side)


def oracle_append(h, spec, slot_mapping):
    """The oracle's append for one layer's host copies: (k, v, k_scales, v_scales)."""
    kc, vc = h["k_cache"], h["v_cache"]
    ks, vs = h.get("k_scales"), h.get("v_scales")
    if spec.append:
        if spec.quantised:
            gran = lambda tok: "token" if tok else "block"
            if spec.k_quantised:
                kn = oracle.stored_to_f64(h["k_new"], spec.q_dtype).astype(np.float32)
                kc, ks = oracle.kv_append_quant(kc, ks, kn, slot_mapping, code=spec.kv_dtype,
                                                first_write=False,
                                                channel_scales=h.get("k_channel_scales"),
                                                granularity=gran(spec.k_scale_tok))
            else:
                kc = oracle.kv_append_bits(kc, h["k_new"], slot_mapping)
            vn = oracle.stored_to_f64(h["v_new"], spec.q_dtype).astype(np.float32)
            vc, vs = oracle.kv_append_quant(vc, vs, vn, slot_mapping, code=spec.v_tag,
                                            first_write=False, granularity=gran(spec.v_scale_tok))
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
    if "k_channel_scales" in x:
        h["k_channel_scales"] = host_storage(x["k_channel_scales"])
    if "sink_k" in x:
        h["sink_k"] = host_storage(x["sink_k"][layer])
        h["sink_v"] = host_storage(x["sink_v"][layer])
        h["sink_tiles_of_seq"] = host_storage(x["sink_tiles_of_seq"])
        if "sink_slot_mapping" in x:
            h["sink_slot_mapping"] = host_storage(x["sink_slot_mapping"])
    return h


def out_f64(out: torch.Tensor) -> np.ndarray:
    return out.detach().float().cpu().numpy().astype(np.float64)


def half_ulp(ref: np.ndarray, tag: str) -> np.ndarray:
    """Half a unit in the last place of the output type at |ref|: the one
    rounding of the result to that type, which no kernel can avoid."""
    mant = {"f32": 23, "f16": 10, "bf16": 7}[tag]
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126)))
    return np.ldexp(0.5, (e - mant).astype(int))


def parity_err(got: np.ndarray, ref: np.ndarray, tag: str, tol: float) -> float:
    """The figure compared with `tol`: max |got - ref|, raw.  Only where the
    output type's half-ulp at |ref| is itself larger than `tol` (bf16 with
    |ref| >= 4, f16 with |ref| >= 32: the full-precision sink tiles draw
    such values) is that one final rounding of the result to the output type
    taken off the element's error, since no kernel can avoid it."""
    if not got.size:
        return 0.0
    hu = half_ulp(ref, tag)
    return float(np.max(np.abs(got - ref) - np.where(hu > tol, hu, 0.0)))


def max_err(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0
