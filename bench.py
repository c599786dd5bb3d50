#!/usr/bin/env python3
"""Decode-step benchmark: paged decode attention KV GB/s on one MI355X.

One step = for every layer: kv_append of each sequence's new token, then
paged_decode_attn over all cached tokens (the whole hot path), on synthetic
seeded inputs already resident in HBM.  Default workload: the 70B-shaped
fp16 step (80 layers, 64 sequences x 4096 tokens, 64 query / 8 KV heads,
head_dim 128).

Prints ONE JSON line.  `value` = KV bytes the attention streams per step
divided by the step's wall time (append included).  `roofline` describes the
attention launch: algorithmic bytes per launch / mean launch duration from
HIP events recorded on the launch stream inside the timed region, against
the 8 TB/s HBM peak.  `cpu_baseline` is the float64 numpy oracle timed on
this host over a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cpu-seconds S]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attention KV GB/s and % of MI355X HBM peak (1 GPU)"
ELT = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_bytes(spec, lay):
    """Algorithmic bytes of one attention launch (one layer).

    K and V of every attended (token, KV head) once, plus q, out, the block
    table entries and lengths read, and the fp8 scales of every attended
    (block, KV head)."""
    L = lay.context_lens.astype(int)
    nblk = -(-L // 16)
    kv = int(L.sum()) * spec.num_kv_heads * spec.head_dim * ELT[spec.kv_dtype] * 2
    q = spec.num_seqs * spec.num_q_heads * spec.head_dim * ELT[spec.q_dtype]
    out = spec.num_seqs * spec.num_q_heads * spec.head_dim * ELT[spec.out_dtype]
    meta = int(nblk.sum()) * 4 + spec.num_seqs * 4
    scales = int(nblk.sum()) * spec.num_kv_heads * 4 * 2 if spec.kv_dtype == "fp8_e4m3" else 0
    return kv, kv + q + out + meta + scales


def cpu_baseline(spec, lay, x, budget_s: float):
    """Time the oracle on whole sequences of layer 0 until ~budget_s of CPU work."""
    import numpy as np
    import torch

    import oracle
    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))
    dev = x["q"].device

    def host(t):
        t = t.detach().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    nblk = -(-lay.context_lens.astype(int) // 16)
    done_bytes, elapsed, seqs = 0, 0.0, 0
    with threadpool_limits(limits=cores):
        for b in range(spec.num_seqs):
            used = lay.block_tables[b, : nblk[b]].astype(np.int64)
            idx = torch.from_numpy(used).to(dev)
            kc = host(x["k_cache"][0].index_select(0, idx))
            vc = host(x["v_cache"][0].index_select(0, idx))
            table = np.arange(len(used), dtype=np.int32)[None, :]
            lens = lay.context_lens[b : b + 1]
            q = host(x["q"][0][b : b + 1])
            kw = {}
            if "k_scales" in x:
                kw = dict(k_scales=host(x["k_scales"][0].index_select(0, idx)),
                          v_scales=host(x["v_scales"][0].index_select(0, idx)))
            t0 = time.perf_counter()
            if spec.append:
                s = int(lay.slot_mapping[b])
                slot = np.array([int(np.nonzero(used == s // 16)[0][0]) * 16 + s % 16])
                kc = oracle.kv_append_bits(kc, host(x["k_new"][0][b : b + 1]), slot)
                vc = oracle.kv_append_bits(vc, host(x["v_new"][0][b : b + 1]), slot)
            oracle.paged_decode_attention(q, kc, vc, table, lens, spec.scale, q_tag=spec.q_dtype,
                                          kv_tag=spec.kv_dtype, **kw)
            elapsed += time.perf_counter() - t0
            done_bytes += int(lens[0]) * spec.num_kv_heads * spec.head_dim * ELT[spec.kv_dtype] * 2
            seqs += 1
            if elapsed >= budget_s:
                break
    return {
        "value": round(done_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"float64 numpy oracle (append + attention), layer 0, {seqs} of "
                  f"{spec.num_seqs} sequences, all {spec.num_q_heads} query heads; "
                  f"{done_bytes / 1e9:.3f} GB of K/V in {elapsed:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama70b_f16_80l")
    ap.add_argument("--partition-blocks", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="0 skips the CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_56_amd as pkv
    from workloads import WORKLOADS, build_layout, make_device_inputs

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pkv.load_library()
    spec = WORKLOADS[args.workload]
    lay = build_layout(spec)
    log(f"[bench] {spec.description}: generating inputs on the device")
    x = make_device_inputs(lay, "cuda")
    torch.cuda.synchronize()
    nl = spec.num_layers
    odt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[spec.out_dtype]
    outs = torch.empty((nl, spec.num_seqs, spec.num_q_heads, spec.head_dim), dtype=odt, device=dev)
    dims = pkv.decode_dims(x["q"][0], x["k_cache"][0], x["block_tables"], outs[0], args.partition_blocks)
    nparts = pkv.decode_num_partitions(dims)
    ws_bytes = pkv.decode_workspace_bytes(dims)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    fp8 = spec.kv_dtype == "fp8_e4m3"

    def step(ev=None):
        for layer in range(nl):
            kc, vc = x["k_cache"][layer], x["v_cache"][layer]
            if spec.append:
                pkv.kv_append(x["k_new"][layer], x["v_new"][layer], x["slot_mapping"], kc, vc)
            if ev is not None:
                ev[layer][0].record()
            kw = dict(k_scales=x["k_scales"][layer], v_scales=x["v_scales"][layer]) if fp8 else {}
            pkv.paged_decode_attn(x["q"][layer], kc, vc, x["block_tables"], x["context_lens"],
                                  spec.scale, outs[layer], workspace=ws,
                                  partition_blocks=args.partition_blocks, **kw)
            if ev is not None:
                ev[layer][1].record()

    log(f"[bench] warmup {args.warmup} steps (partitions per sequence: {nparts})")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nl)]
              for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = np.array([[e[0].elapsed_time(e[1]) for e in row] for row in events])
    mean_launch_s = float(launch_ms.mean()) / 1e3

    kv_bytes, alg_bytes = attention_bytes(spec, lay)
    value = kv_bytes * nl / (ms_per_step / 1e3) / 1e9
    achieved = alg_bytes / mean_launch_s / 1e9
    kernel = "decode_partition_kernel" + ("+lse_merge_kernel" if nparts > 1 else "")
    log(f"[bench] {ms_per_step:.3f} ms/step; attention launch {mean_launch_s * 1e6:.1f} us "
        f"-> {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of peak)")

    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(spec, lay, x, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8_e4m3": "fp8_e4m3"}[spec.kv_dtype],
        "data": "synthetic",
        "config": {
            "workload": spec.name,
            "layers": nl,
            "num_seqs": spec.num_seqs,
            "context_lens": "4096 each" if spec.name == "llama70b_f16_80l" else "see workloads/specs.py",
            "q_heads": spec.num_q_heads,
            "kv_heads": spec.num_kv_heads,
            "head_dim": spec.head_dim,
            "block_size": 16,
            "partitions": nparts,
            "kv_bytes_per_step": kv_bytes * nl,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "bytes_per_launch": alg_bytes,
            "mean_launch_us": round(mean_launch_s * 1e6, 2),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
