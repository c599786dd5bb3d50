#!/usr/bin/env python3
"""Decode-step benchmark: paged decode attention KV GB/s on one MI355X.

One step = for every layer: kv_append of each sequence's new token (8-bit
caches quantise it on write), then paged_decode_attn over all cached tokens
(the whole hot path), on synthetic
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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CALIB_COPY_BYTES = 512 * 2**20
CALIB_COPY_KERNEL = "__amd_rocclr_copyBuffer"
PROBE_KERNEL = "pkv::hbm_read_kernel"
ATTN_KERNEL = "pkv::decode_partition_kernel"
CSRC = os.path.join(ROOT, "paged_kv_cache_56_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "paged decode attention KV GB/s and % of MI355X HBM peak (1 GPU)"
ELT = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1, "int8": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attended(L: int, window: int, sinks: int):
    """Positions a length-L sequence attends (the oracle's definition, restated
    here so the byte count does not import the oracle)."""
    if window <= 0 or L <= window:
        return range(L)
    return sorted(set(range(min(sinks, L))) | set(range(L - window, L)))


def attention_bytes(spec, lay, window: int = 0, sinks: int = 0):
    """Algorithmic bytes of one attention launch (one layer).

    K and V of every attended (token, KV head) once -- a physical block that
    several sequences share (a common prefix) is counted once, since the
    method needs to stream it only once -- plus q, out, the block table
    entries and lengths read, the 8-bit scales of every attended (block, KV
    head) and K's channel factors.  Returns (K/V bytes, all algorithmic bytes, logical K/V bytes
    counting shared blocks once per sequence)."""
    L = lay.context_lens.astype(int)
    per_token = spec.num_kv_heads * spec.head_dim * (ELT[spec.kv_dtype] + ELT[spec.v_tag])
    side_token = spec.num_kv_heads * spec.head_dim * 2 * ELT[spec.q_dtype]   # full-precision sinks
    S = spec.fp_sinks
    logical = 0
    side = 0
    used = {}                        # physical block -> attended token offsets
    for b in range(spec.num_seqs):
        pos = attended(int(L[b]), window, S or sinks)
        logical += len(pos) * per_token
        for p in pos:
            if p < S:
                side += side_token
                continue
            used.setdefault(int(lay.block_tables[b, p // 16]), set()).add(p % 16)
    kv = sum(len(v) for v in used.values()) * per_token + side
    nblk = np.array([len({p // 16 for p in attended(int(l), window, sinks)}) for l in L])
    q = spec.num_seqs * spec.num_q_heads * spec.head_dim * ELT[spec.q_dtype]
    out = spec.num_seqs * spec.num_q_heads * spec.head_dim * ELT[spec.out_dtype]
    meta = int(nblk.sum()) * 4 + spec.num_seqs * 4
    # 8-bit scales of every attended (block, KV head): one fp32, or 16 per-token ones
    per_scale = lambda tok: int(nblk.sum()) * spec.num_kv_heads * 4 * (16 if tok else 1)
    scales = ((per_scale(spec.k_scale_tok) if spec.k_quantised else 0) +
              (per_scale(spec.v_scale_tok) if spec.v_tag in ("fp8_e4m3", "int8") else 0))
    chan = spec.num_kv_heads * spec.head_dim * 4 if spec.k_outliers else 0
    return kv, kv + q + out + meta + scales + chan, logical


PARITY_TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2, "fp8_e4m3": 5e-2, "int8": 5e-2}


def cpu_baseline(spec, lay, x, budget_s: float, outs=None):
    """Time the oracle on whole sequences (layer 0, then layer 1, ...) until
    about budget_s seconds of CPU work have been spent.

    The oracle's result for each (layer, sequence) it ran is also compared
    with the GPU's output for that layer from the last timed step (`outs`):
    the inputs are the caches as the timed steps left them (every step
    appends the same new token to the same slot, so the oracle's own append
    on top of them must change nothing), and the largest absolute difference
    is reported next to the tolerance for the cache format."""
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
    max_err = 0.0
    order = [(layer, b) for layer in range(x["k_cache"].shape[0]) for b in range(spec.num_seqs)]
    with threadpool_limits(limits=cores):
        for layer, b in order:
            used = lay.block_tables[b, : nblk[b]].astype(np.int64)
            idx = torch.from_numpy(used).to(dev)
            kc = host(x["k_cache"][layer].index_select(0, idx))
            vc = host(x["v_cache"][layer].index_select(0, idx))
            table = np.arange(len(used), dtype=np.int32)[None, :]
            lens = lay.context_lens[b : b + 1]
            q = host(x["q"][layer][b : b + 1])
            kw = {}
            for name in ("k_scales", "v_scales"):
                if name in x:
                    kw[name] = host(x[name][layer].index_select(0, idx))
            chan = host(x["k_channel_scales"]) if "k_channel_scales" in x else None
            if spec.fp_sinks:
                tile = int(x["sink_tiles_of_seq"][b])
                kw.update(sink_k=host(x["sink_k"][layer][tile:tile + 1]),
                          sink_v=host(x["sink_v"][layer][tile:tile + 1]),
                          sink_blocks=np.zeros(1, np.int64), sinks=spec.fp_sinks)
            t0 = time.perf_counter()
            if spec.append:
                s = int(lay.slot_mapping[b])
                slot = np.array([int(np.nonzero(used == s // 16)[0][0]) * 16 + s % 16])
                kn = host(x["k_new"][layer][b : b + 1])
                vn = host(x["v_new"][layer][b : b + 1])
                gran = lambda tok: "token" if tok else "block"
                if spec.quantised:
                    if spec.k_quantised:
                        kn = oracle.stored_to_f64(kn, spec.q_dtype).astype(np.float32)
                        kc, kw["k_scales"] = oracle.kv_append_quant(kc, kw["k_scales"], kn, slot,
                                                                    code=spec.kv_dtype, first_write=False,
                                                                    channel_scales=chan,
                                                                    granularity=gran(spec.k_scale_tok))
                    else:
                        kc = oracle.kv_append_bits(kc, kn, slot)
                    vn = oracle.stored_to_f64(vn, spec.q_dtype).astype(np.float32)
                    vc, kw["v_scales"] = oracle.kv_append_quant(vc, kw["v_scales"], vn, slot,
                                                                code=spec.v_tag, first_write=False,
                                                                granularity=gran(spec.v_scale_tok))
                else:
                    kc = oracle.kv_append_bits(kc, kn, slot)
                    vc = oracle.kv_append_bits(vc, vn, slot)
            ref = oracle.paged_decode_attention(q, kc, vc, table, lens, spec.scale, q_tag=spec.q_dtype,
                                                kv_tag=spec.kv_dtype, v_tag=spec.v_tag,
                                                k_channel_scales=chan, **kw)
            elapsed += time.perf_counter() - t0
            if outs is not None:
                got = outs[layer][b].float().cpu().numpy().astype(np.float64)
                max_err = max(max_err, float(np.abs(got - ref[0]).max()))
            done_bytes += int(lens[0]) * spec.num_kv_heads * spec.head_dim * (ELT[spec.kv_dtype] +
                                                                              ELT[spec.v_tag])
            seqs += 1
            if elapsed >= budget_s:
                break
    rec = {
        "value": round(done_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"float64 numpy oracle (append + attention) on {seqs} (layer, sequence) pairs "
                  f"of {x['k_cache'].shape[0] * spec.num_seqs}, all {spec.num_q_heads} query heads each; "
                  f"{done_bytes / 1e9:.3f} GB of K/V in {elapsed:.1f} s",
    }
    if outs is not None:
        rec["max_abs_err_vs_gpu"] = max_err
        rec["tol"] = PARITY_TOL[spec.kv_dtype]
    return rec


def read_probe(dev, gib: int = 4):
    """Plain streaming read (the library's hbm_read_probe) over `gib` GiB: the
    rate a read-only kernel gets from HBM on this device.  Best of a few grid
    sizes.  Also runs one 512 MiB device copy, a kernel of known traffic (512
    MiB read + 512 MiB written) that counter runs use to scale FETCH_SIZE and
    WRITE_SIZE."""
    import torch

    import paged_kv_cache_56_amd as pkv

    buf = torch.empty(gib * 2**30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    best = 0.0
    for wgs in (512, 1024, 2048, 4096):
        sink = torch.zeros(wgs, dtype=torch.int32, device=dev)
        pkv.hbm_read_probe(buf, sink)            # warm
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            pkv.hbm_read_probe(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 5 * buf.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del buf
    src = torch.ones(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    return {"gbs": best, "bytes": gib * 2**30}


def grouped_probe_rows(lay, group_pieces: int):
    """Block-table rows and lengths whose plain per-sequence reading is the
    unique traffic of a shared-prefix launch: each group's shared blocks cut
    into `group_pieces` equal pieces (one row each, read once, and first, as
    the group pass's workgroups lead the launch), then every sequence's
    blocks after its group's shared ones.  Host-side bookkeeping only."""
    tab, lens = lay.block_tables, lay.context_lens.astype(np.int64)
    B, maxb = tab.shape
    skip = np.zeros(B, dtype=np.int64)
    rows, rlens = [], []
    for g in range(len(lay.group_blocks)):
        s0, s1 = int(lay.group_starts[g]), int(lay.group_starts[g + 1])
        nb = int(lay.group_blocks[g])
        if s1 <= s0 or nb <= 0:
            continue
        skip[s0:s1] = nb
        pb = -(-nb // max(1, group_pieces))
        for j0 in range(0, nb, pb):
            j1 = min(j0 + pb, nb)
            r = np.zeros(maxb, dtype=np.int32)
            r[:j1 - j0] = tab[s0, j0:j1]
            rows.append(r)
            rlens.append((j1 - j0) * 16)
    for b in range(B):
        r = np.zeros(maxb, dtype=np.int32)
        k = int(skip[b])
        r[:maxb - k] = tab[b, k:]
        rows.append(r)
        rlens.append(int(lens[b]) - 16 * k)
    return np.stack(rows).astype(np.int32), np.array(rlens, dtype=np.int32)


def pattern_probe(x, lay, spec, dims, layers: int, launches: int, stride: int, rows=None):
    """The attention launch's access pattern without its arithmetic (the
    library's paged_read_probe: same grid, tables, LDS-DMA K ring and V
    register loads) on the same caches, launched like the attention calls
    (layer after layer, HIP events around every `stride`-th launch).  With
    `rows` = (block tables, lengths, dims) the probe reads those rows instead
    (a shared-prefix launch's unique blocks).
    Returns its mean launch time and K/V bytes per launch."""
    import torch

    import paged_kv_cache_56_amd as pkv

    tables, lens = x["block_tables"], x["context_lens"]
    nblk = -(-lay.context_lens.astype(np.int64) // 16)
    if rows is not None:
        tab_np, lens_np, dims = rows
        tables = torch.from_numpy(tab_np).to(x["q"].device)
        lens = torch.from_numpy(lens_np).to(x["q"].device)
        nblk = -(-lens_np.astype(np.int64) // 16)
    P = pkv.decode_num_partitions(dims)
    sink = torch.zeros(dims.num_seqs * spec.num_kv_heads * P, dtype=torch.int32, device=x["q"].device)
    for layer in range(layers):                   # warm
        pkv.paged_read_probe(x["k_cache"][layer], x["v_cache"][layer], tables, lens, dims, sink)
    torch.cuda.synchronize()
    ev = []
    for k in range(launches):
        layer = k % layers
        timed = k % stride == 0
        if timed:
            e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            e[0].record()
        pkv.paged_read_probe(x["k_cache"][layer], x["v_cache"][layer], tables, lens, dims, sink)
        if timed:
            e[1].record()
            ev.append(e)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    tile = 16 * spec.head_dim * (ELT[spec.kv_dtype] + ELT[spec.v_tag])
    return us, int(nblk.sum()) * spec.num_kv_heads * tile


def copy_blocks_rate(x, spec, pairs: int):
    """Copy-on-write block copies on layer 0's caches: `pairs` random
    (src, dst) pairs with distinct destinations, each moving a whole block of
    K and V (every head) -- read once, written once."""
    import torch

    import paged_kv_cache_56_amd as pkv

    kc, vc = x["k_cache"][0], x["v_cache"][0]
    nb = kc.shape[0]
    pairs = min(pairs, nb // 2, 65535)
    g = torch.Generator().manual_seed(spec.seed)
    perm = torch.randperm(nb, generator=g)
    src = perm[:pairs].to(torch.int32).to(kc.device)
    dst = perm[pairs:2 * pairs].to(torch.int32).to(kc.device)
    kw = dict(k_scales=x["k_scales"][0], v_scales=x["v_scales"][0]) if "k_scales" in x else {}
    pkv.copy_blocks(kc, vc, src, dst, **kw)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        pkv.copy_blocks(kc, vc, src, dst, **kw)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / reps
    moved = 2 * pairs * kc[0].numel() * kc.element_size() * 2      # K and V, read + write
    return {"pairs": pairs, "block_bytes": kc[0].numel() * kc.element_size(), "us": round(s * 1e6, 2),
            "gbs": round(moved / s / 1e9, 1)}


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that
    comment edits do not count as kernel changes."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_sha() -> str:
    """sha256 over the code (comments dropped) of the HIP sources and headers
    the library is built from."""
    import hashlib

    h = hashlib.sha256()
    for fn in sorted(os.listdir(CSRC)):
        if fn.endswith((".hip", ".h", ".cpp")):
            h.update(fn.encode())
            h.update(_code_only(open(os.path.join(CSRC, fn)).read()).encode())
    h.update(_code_only(open(os.path.join(ROOT, "include", "pagedkv.h")).read()).encode())
    return h.hexdigest()[:16]


def _csv_rows(path):
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_counters(fetch_csv, write_csv, stats_csv, workload, probe_gib, out_md, command,
                       kernel=ATTN_KERNEL, layers=0):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench plus
    its --kernel-trace --stats run into the traffic summary bench.py reports.

    Scale factors come from kernels of known traffic in the same runs: the
    read probe (probe_gib GiB read) for FETCH_SIZE and a 512 MiB copy for
    WRITE_SIZE (and as a FETCH_SIZE cross-check)."""
    import statistics

    def per_kernel(rows, counter):
        d = {}
        for r in rows:
            if r["Counter_Name"] == counter:
                d.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return d

    def calib_copy(rows, counter):
        # the 512 MiB copy read_probe() makes: the first copy dispatched after
        # the last read-probe dispatch (input generation makes other copies,
        # some larger)
        rows = sorted((r for r in rows if r["Counter_Name"] == counter), key=lambda r: int(r["Dispatch_Id"]))
        last = max(i for i, r in enumerate(rows) if PROBE_KERNEL in r["Kernel_Name"])
        return next(float(r["Counter_Value"]) * 1024.0 for r in rows[last + 1:]
                    if r["Kernel_Name"].startswith(CALIB_COPY_KERNEL))

    fetch_rows, write_rows = _csv_rows(fetch_csv), _csv_rows(write_csv)
    fetch = per_kernel(fetch_rows, "FETCH_SIZE")
    write = per_kernel(write_rows, "WRITE_SIZE")
    pick = lambda d, key: [v for k, vals in d.items() if k.startswith(key) or key in k for v in vals]
    probe_f = max(pick(fetch, PROBE_KERNEL))
    copy_f = calib_copy(fetch_rows, "FETCH_SIZE")
    copy_w = calib_copy(write_rows, "WRITE_SIZE")
    fetch_scale = probe_gib * 2**30 / probe_f
    write_scale = CALIB_COPY_BYTES / copy_w
    attn_f = statistics.mean(pick(fetch, kernel)) * fetch_scale
    attn_w = statistics.mean(pick(write, kernel)) * write_scale
    stats = [r for r in _csv_rows(stats_csv)]
    top = sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:6]
    attn = [r for r in stats if kernel in r["Name"]]
    rec = {
        "workload": workload,
        "layers": layers or None,
        "kernel": kernel,
        "kernel_source_sha": kernel_source_sha(),
        "fetch_bytes_per_launch": round(attn_f),
        "write_bytes_per_launch": round(attn_w),
        "traffic_bytes_per_launch": round(attn_f + attn_w),
        "fetch_scale": round(fetch_scale, 4),
        "fetch_scale_check_copy": round(CALIB_COPY_BYTES / copy_f, 4),
        "write_scale": round(write_scale, 4),
        "trace_mean_launch_us": round(float(attn[0]["AverageNs"]) / 1e3, 2) if attn else None,
        "trace_calls": int(attn[0]["Calls"]) if attn else 0,
    }
    lines = [
        f"# {kernel} on {workload}: rocprofv3 summary",
        "",
        "Commands (run from the repository root on one MI355X, `export TMPDIR=/tmp`):",
        "",
        "```",
        *command,
        "```",
        "",
        "## Kernel trace (--kernel-trace --stats), top kernels by total time",
        "",
        "| kernel | calls | mean us | min us | max us | share |",
        "|---|---|---|---|---|---|",
    ]
    for r in top:
        name = r["Name"].replace("|", "/")
        name = name if len(name) < 90 else name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    lines += [
        "",
        "## HBM traffic (--pmc FETCH_SIZE, --pmc WRITE_SIZE; one run each)",
        "",
        f"FETCH_SIZE reads {probe_f / 2**30:.3f} GiB for the read probe that reads {probe_gib} GiB "
        f"(scale {fetch_scale:.4f}); the 512 MiB copy gives {CALIB_COPY_BYTES / copy_f:.4f}.  "
        f"WRITE_SIZE reads {copy_w / 2**20:.1f} MiB for the 512 MiB copy (scale {write_scale:.4f}).",
        "",
        "```json",
        json.dumps(rec, indent=1),
        "```",
    ]
    os.makedirs(os.path.dirname(out_md), exist_ok=True)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return rec


def summarize_trace(stats_csv, workload, out_md, command, kernel=ATTN_KERNEL):
    """A rocprofv3 --kernel-trace --stats summary (top kernels) for one workload."""
    stats = _csv_rows(stats_csv)
    top = sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:8]
    attn = [r for r in stats if kernel in r["Name"]]
    lines = [f"# {kernel} on {workload}: rocprofv3 kernel trace", "",
             "Command (run from the repository root on one MI355X, `export TMPDIR=/tmp`):", "",
             "```", *command, "```", "",
             "| kernel | calls | mean us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in top:
        name = r["Name"].replace("|", "/")
        name = name if len(name) < 90 else name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    rec = {"workload": workload, "kernel": kernel, "kernel_source_sha": kernel_source_sha(),
           "trace_mean_launch_us": round(float(attn[0]["AverageNs"]) / 1e3, 2) if attn else None,
           "trace_calls": int(attn[0]["Calls"]) if attn else 0}
    lines += ["", "```json", json.dumps(rec, indent=1), "```"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return rec


def traffic_for(workload: str, kernel: str = "decode_partition_kernel", layers: int = 0):
    """Counter-measured bytes per attention launch, if taken on these sources
    with the same layer count (a one-layer workload re-read back to back is
    partly served from the last-level cache; several layers read cold)."""
    import re

    path = os.path.join(PROFILES, f"{kernel}__{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    if layers and rec.get("layers") not in (None, layers):
        return None
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (default: enough for >= 200 attention launches, at least 10)")
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed steps first (default: enough for >= 100 launches, at least 3); "
                         "the GPU needs a few dozen launches to reach its steady clocks")
    ap.add_argument("--workload", default="llama70b_f16_80l")
    ap.add_argument("--layers", type=int, default=0,
                    help="layers per step, each with its own cache (0: the workload's own count); "
                         "several copies of a one-layer workload make every launch read cold data, "
                         "as in a model with many layers")
    ap.add_argument("--partition-blocks", type=int, default=0)
    ap.add_argument("--window", type=int, default=0, help="sliding window W (0 = whole context)")
    ap.add_argument("--sinks", type=int, default=0, help="attention-sink tokens kept with a window")
    ap.add_argument("--fp-sinks", type=int, default=0,
                    help="8-bit workloads: keep this many leading tokens in full-precision side tiles")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="0 skips the CPU baseline")
    ap.add_argument("--copy-pairs", type=int, default=0,
                    help="also time copy-on-write copies of this many random block pairs")
    ap.add_argument("--event-stride", type=int, default=8,
                    help="bracket every N-th attention launch with HIP events (1 = all)")
    ap.add_argument("--separate-append", action="store_true",
                    help="append with its own launch instead of inside the attention launch")
    ap.add_argument("--no-groups", action="store_true",
                    help="attend shared prefixes per sequence instead of once per group")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the plain-read bandwidth probe and the copy used to calibrate counters")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "STATS_CSV"),
                    help="write profiles/decode_partition_kernel__<workload>.md from rocprofv3 output and exit")
    ap.add_argument("--summarize-trace", metavar="STATS_CSV",
                    help="write profiles/<kernel>__<workload>__trace.md from a rocprofv3 "
                         "--kernel-trace --stats run and exit")
    ap.add_argument("--trace-kernel", default=ATTN_KERNEL,
                    help="kernel whose mean launch --summarize-trace records")
    ap.add_argument("--command", action="append", default=[],
                    help="(with --summarize-counters) a command line to record in the summary")
    args = ap.parse_args()
    if args.summarize_trace:
        out = os.path.join(PROFILES, f"{args.trace_kernel.split('::')[-1]}__{args.workload}__trace.md")
        print(json.dumps(summarize_trace(args.summarize_trace, args.workload, out, args.command,
                                         args.trace_kernel)))
        return
    if args.summarize_counters:
        out = os.path.join(PROFILES, f"{args.trace_kernel.split('::')[-1]}__{args.workload}.md")
        rec = summarize_counters(*args.summarize_counters, args.workload, 4, out, args.command,
                                 args.trace_kernel, args.layers)
        print(json.dumps(rec))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_56_amd as pkv
    from workloads import WORKLOADS, build_layout, make_device_inputs, scaled

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pkv.load_library()
    spec = WORKLOADS[args.workload]
    layers = args.layers if args.layers > 0 else spec.num_layers
    if args.warmup < 0:
        args.warmup = max(3, -(-100 // layers))
    if args.steps <= 0:
        args.steps = max(10, -(-200 // layers))
    if args.fp_sinks:
        spec = scaled(spec, fp_sinks=args.fp_sinks)
        args.sinks = args.fp_sinks
    lay = build_layout(spec)
    log(f"[bench] {spec.description}: generating inputs on the device")
    x = make_device_inputs(lay, "cuda", layers)
    torch.cuda.synchronize()
    nl = x["k_cache"].shape[0]
    odt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[spec.out_dtype]
    outs = torch.empty((nl, spec.num_seqs, spec.num_q_heads, spec.head_dim), dtype=odt, device=dev)
    # a scheduler knows its batch's lengths on the host: pass their block count
    # so the split plan can balance uneven sequences
    total_blocks = int((-(-lay.context_lens.astype(np.int64) // 16)).sum())
    # shared prefixes: read once per group (the scheduler knows the groups)
    # (16-bit caches, or K and V of one 8-bit format with per-block scales,
    # a 16-bit q and out of one type, head_dim 128)
    group_ok = spec.kv_dtype in ("f16", "bf16") or (
        spec.k_quantised and spec.v_tag == spec.kv_dtype and not spec.k_outliers and not spec.fp_sinks
        and not (spec.k_scale_tok or spec.v_scale_tok) and spec.q_dtype == spec.out_dtype
        and spec.q_dtype in ("f16", "bf16") and spec.head_dim == 128)
    grouped = (lay.group_starts is not None and not args.no_groups and args.window == 0 and group_ok)
    gkw = {}
    if grouped:
        gkw = dict(prefix_group_starts=x["group_starts"], prefix_group_blocks=x["group_blocks"],
                   prefix_max_seqs=int(np.diff(lay.group_starts).max()),
                   prefix_max_blocks=int(lay.group_blocks.max()))
    dims = pkv.decode_dims(x["q"][0], x["k_cache"][0], x["block_tables"], outs[0], args.partition_blocks,
                           args.window, args.sinks, bool(spec.fp_sinks), total_blocks,
                           len(lay.group_blocks) if grouped else 0, gkw.get("prefix_max_seqs", 0),
                           gkw.get("prefix_max_blocks", 0))
    nparts = pkv.decode_num_partitions(dims)
    ws_bytes = pkv.decode_workspace_bytes(dims)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    chan = x.get("k_channel_scales")
    both_fp8 = (spec.kv_dtype == spec.v_tag == "fp8_e4m3" and chan is None and not spec.fp_sinks
                and not (spec.k_scale_tok or spec.v_scale_tok))
    # the append rides in the attention launch (8-bit caches: quantised there,
    # with the blocks' given scales or per-token scales); not with sink tiles
    fused = spec.append and not spec.fp_sinks and not args.separate_append

    def step(ev=None):
        for layer in range(nl):
            kc, vc = x["k_cache"][layer], x["v_cache"][layer]
            kw = {}
            if spec.quantised:
                kw = dict(v_scales=x["v_scales"][layer])
                if spec.k_quantised:
                    kw["k_scales"] = x["k_scales"][layer]
                if chan is not None:
                    kw["k_channel_scales"] = chan
            if spec.fp_sinks:
                kw.update(sink_k=x["sink_k"][layer], sink_v=x["sink_v"][layer],
                          sink_tiles_of_seq=x["sink_tiles_of_seq"])
                if spec.append:
                    pkv.kv_append(x["k_new"][layer], x["v_new"][layer], x["sink_slot_mapping"],
                                  x["sink_k"][layer], x["sink_v"][layer])
            if spec.append and fused:
                pass                                # written by the attention launch
            elif spec.append and both_fp8:
                pkv.kv_append_fp8(x["k_new"][layer], x["v_new"][layer], x["slot_mapping"], kc, vc,
                                  kw["k_scales"], kw["v_scales"])
            elif spec.append and spec.quantised:
                if spec.k_quantised:
                    pkv.kv_append_quant(x["k_new"][layer], x["slot_mapping"], kc, kw["k_scales"],
                                        channel_scales=chan)
                else:                               # a 16-bit K: a bit copy of K alone
                    pkv.kv_append(x["k_new"][layer], None, x["slot_mapping"], kc, None)
                pkv.kv_append_quant(x["v_new"][layer], x["slot_mapping"], vc, kw["v_scales"])
            elif spec.append:
                pkv.kv_append(x["k_new"][layer], x["v_new"][layer], x["slot_mapping"], kc, vc)
            if ev is not None and layer in ev:
                ev[layer][0].record()
            if fused:
                pkv.paged_decode_step(x["k_new"][layer], x["v_new"][layer], x["slot_mapping"], x["q"][layer],
                                      kc, vc, x["block_tables"], x["context_lens"], spec.scale, outs[layer],
                                      workspace=ws, partition_blocks=args.partition_blocks,
                                      window=args.window, sinks=args.sinks, total_blocks=total_blocks,
                                      **gkw, **kw)
            else:
                pkv.paged_decode_attn(x["q"][layer], kc, vc, x["block_tables"], x["context_lens"],
                                      spec.scale, outs[layer], workspace=ws,
                                      partition_blocks=args.partition_blocks, window=args.window,
                                      sinks=args.sinks, total_blocks=total_blocks, **kw, **gkw)
            if ev is not None and layer in ev:
                ev[layer][1].record()

    log(f"[bench] warmup {args.warmup} steps (partitions per sequence: {nparts})")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # HIP events bracket a sample of the launches (every event_stride-th,
    # rotating over layers): each event is a packet the command processor
    # handles between kernels, so bracketing all of them would lengthen the
    # step that `value` is computed from.
    stride = max(1, args.event_stride)
    events = [{layer: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for layer in range(nl) if (k + layer) % stride == 0} for k in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = np.array([e[0].elapsed_time(e[1]) for row in events for e in row.values()])
    mean_launch_s = float(launch_ms.mean()) / 1e3

    kv_bytes, alg_bytes, logical_bytes = attention_bytes(spec, lay, args.window, args.sinks)
    if fused:
        # the launch also reads each new K/V row (q's dtype for an 8-bit cache)
        # and writes it to its slot, with its per-token scale where there is one
        rows = spec.num_seqs * spec.num_kv_heads
        src = ELT[spec.q_dtype] if spec.quantised else ELT[spec.kv_dtype]
        alg_bytes += rows * spec.head_dim * (2 * src + ELT[spec.kv_dtype] + ELT[spec.v_tag])
        alg_bytes += rows * 4 * (int(spec.k_scale_tok) + int(spec.v_scale_tok))
    value = kv_bytes * nl / (ms_per_step / 1e3) / 1e9
    achieved = alg_bytes / mean_launch_s / 1e9
    kernel = ("decode_group_kernel" if grouped else "decode_partition_kernel") + (
        "+lse_merge_kernel" if (nparts > 1 or grouped) else "")
    trec = (traffic_for(spec.name, kernel.split("+")[0], nl) if args.window == 0 and not args.fp_sinks
            else None)
    traffic = None if trec is None else trec["traffic_bytes_per_launch"]
    log(f"[bench] {ms_per_step:.3f} ms/step; attention launch {mean_launch_s * 1e6:.1f} us "
        f"-> {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of peak)")

    copy_rec = None
    if args.copy_pairs > 0:
        copy_rec = copy_blocks_rate(x, spec, args.copy_pairs)
        log(f"[bench] copy-on-write copies: {copy_rec['pairs']} block pairs, {copy_rec['gbs']:.0f} GB/s")

    pat = None
    if (not args.no_probe and args.window == 0 and not spec.fp_sinks and spec.head_dim == 128
            and ELT[spec.v_tag] <= ELT[spec.kv_dtype] <= 2):
        rows = None
        if grouped:
            # the group pass's pieces per group, from the workspace it is given
            # (a partial result per query row per piece)
            row_b = spec.num_seqs * spec.num_q_heads * (spec.head_dim + 2) * 4
            gpieces = ws_bytes // row_b - nparts
            tab_np, lens_np = grouped_probe_rows(lay, gpieces)
            qd = torch.empty((len(lens_np), spec.num_q_heads, spec.head_dim), dtype=x["q"].dtype, device=dev)
            tb = torch.from_numpy(tab_np)
            pdims = pkv.decode_dims(qd, x["k_cache"][0], tb, qd, args.partition_blocks, 0, 0, False,
                                    int((-(-lens_np.astype(np.int64) // 16)).sum()))
            rows = (tab_np, lens_np, pdims)
            log(f"[bench] access-pattern probe rows: {gpieces} prefix pieces per group + the suffixes "
                f"({pkv.decode_num_partitions(pdims)} partitions per row)")
        pat_us, pat_bytes = pattern_probe(x, lay, spec, dims, nl, max(40, len(launch_ms) * stride), stride,
                                          rows)
        pat = {"us": pat_us, "gbs": pat_bytes / (pat_us / 1e6) / 1e9}
        log(f"[bench] access-pattern probe: {pat_us:.1f} us per launch, {pat['gbs']:.0f} GB/s; the attention "
            f"launch takes {mean_launch_s * 1e6 / pat_us:.3f}x as long")

    probe = None
    if not args.no_probe:
        probe = read_probe(dev)
        log(f"[bench] plain read probe: {probe['gbs']:.0f} GB/s over {probe['bytes'] / 2**30:.0f} GiB")

    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(spec, lay, x, args.cpu_seconds, outs)
        log(f"[bench] GPU output of the last step vs the oracle on the sampled (layer, sequence) "
            f"pairs: max|err| = {cpu['max_abs_err_vs_gpu']:.3e} (tol {cpu['tol']})")

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
        "dtype": spec.kv_dtype if spec.v_tag == spec.kv_dtype else f"{spec.kv_dtype}+{spec.v_tag}",
        "scales": None if not spec.quantised else ("per token" if (spec.k_scale_tok or spec.v_scale_tok)
                                                   else "per block"),
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
            "window": args.window,
            "sinks": args.sinks if (args.window > 0 or spec.fp_sinks) else 0,
            "fp_sinks": spec.fp_sinks,
            "prefix_groups": len(lay.group_blocks) if grouped else 0,
            "append": ("in the attention launch" if fused else "own launch") if spec.append else "none",
            "kv_bytes_per_step": kv_bytes * nl,
            "logical_kv_bytes_per_step": logical_bytes * nl,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": alg_bytes,
            "mean_launch_us": round(mean_launch_s * 1e6, 2),
            "launches_timed": int(launch_ms.size),
            "traffic_over_algorithmic": None if traffic is None else round(traffic / alg_bytes, 4),
            "kernel_source_sha": kernel_source_sha(),
            "read_probe_gbs": None if probe is None else round(probe["gbs"], 1),
            "frac_of_read_probe": None if probe is None else round(achieved / probe["gbs"], 4),
            # the same K/V tiles through the same grid and staging, no arithmetic
            "pattern_probe_us": None if pat is None else round(pat["us"], 2),
            "pattern_probe_gbs": None if pat is None else round(pat["gbs"], 1),
            "frac_of_pattern_probe": None if pat is None else round(pat["us"] / (mean_launch_s * 1e6), 4),
        },
        "cpu_baseline": cpu,
        "max_abs_err": None if cpu is None else cpu["max_abs_err_vs_gpu"],
    }
    if copy_rec is not None:
        rec["copy_blocks"] = copy_rec
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
