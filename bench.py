#!/usr/bin/env python3
"""Benchmark of Slow-Fast decode attention on one MI355X.

A step is one slow-fast cycle of a stack of --layers layers of the workload, each with its own
K/V, logits and indices, run in decode order: token 0 runs the slow step of every layer in turn
(the dense step with fp32 logit write, sfi_dense_decode; the Selector, sfi_select; the
sink-bypass mask when the workload has one, sfi_sink_bypass_mask), then each of the cycle-1
later tokens runs the fast step (sfi_sparse_decode) of every layer in turn, with the recent
window one token further on.  Between two calls on one layer the other layers' calls run, so
repeated reads are not served from the 256 MB Infinity Cache.  Inputs are resident in HBM
before the timed region.

Prints one JSON line.  value = microseconds per decode step of one layer, amortised over the
cycle: stack-cycle time / (cycle * layers), from the host clock around whole stack cycles run
back to back.  roofline = the dense slow step's algorithmic HBM bytes per launch / its mean
time, measured with HIP events on the launch stream inside the timed region (the only events
there).  The per-call breakdown (select, mask, fast) comes from separate instrumented cycles;
spread_us gives p10/p50/p90 over single calls each bracketed by its own events (an event pair
adds about 1.5 us to a call, so these sit above the block means), and dense_nolog_us the dense
step without its logit write.  graph_cycle = the same stack cycle captured once in a HIP graph
and replayed, next to the eager value.
cpu_baseline = the fp64 CPU oracle timed on the host on whole cycles of one layer.
read_yardstick = a plain sequential read of 4 GiB (sfi_stream_read) on the same box; the
rooflines also give the dense and fast rates as a fraction of it, next to the 8 TB/s peak.
fast_roofline.floor = what the fast step's bytes cost without its arithmetic: the same rows read
once by one launch (sfi_gather_read), a launch with almost nothing to do, and a sequential read
of as many bytes, cold in the Infinity Cache (the fastest any one-launch read of them can be).
group_dot = the GQA group's dot products over a layer's key rows on the vector ALUs and on MFMA,
beside a read of the same rows with the same access pattern (sfi_group_dot).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fast/slow decode-attn µs/step + achieved HBM GB/s (% of peak) at 32K–512K ctx"
PEAK_HBM_GBS = 8000.0
# The sources that decide the attention kernels' HBM traffic: the kernels, and the launch plan
# (grid, split lengths) with its constants.  Committed counter figures carry their hash.
ATTN_SRCS = [os.path.join(ROOT, "sparse_kv_attention_dense_amd", "csrc", f)
             for f in ("sfi_attention.hip", "sfi_api.cpp", "sfi_internal.h")]


def attention_sources_sha256() -> str:
    h = hashlib.sha256()
    for path in ATTN_SRCS:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="sink_128k_b4")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layered", action="store_true",
                    help="skip the layer-wise slow-step measurement (sequential vs pipelined)")
    ap.add_argument("--no-spread", action="store_true",
                    help="skip the per-call spread pass (it also runs the dense step without "
                         "logits, which a kernel trace would mix into the dense kernel's stats)")
    ap.add_argument("--no-routed", action="store_true",
                    help="skip the routed fast-step measurement on sink-dominated workloads")
    ap.add_argument("--no-refined", action="store_true",
                    help="skip the full Selector (prior and refinements) measurement")
    ap.add_argument("--no-two-segment", action="store_true",
                    help="skip the Reorg + two-segment fast-step measurement")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the stack cycle replayed from a captured HIP graph")
    ap.add_argument("--context-sweep", action="store_true",
                    help="add dense, Selector and fast-step timings of an 8B-shaped layer at "
                         "contexts of 32K to 512K")
    ap.add_argument("--retention-sweep", action="store_true",
                    help="add dense-vs-sparse timings over retention ratios on a layer shaped "
                         "like the SFI page's retention table (KV 16K, batch 16, 32/8 heads)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed region, copy MIB MiB on the device a few times (a "
                         "known-size reference for rocprofv3 byte counters)")
    return ap.parse_args()


def kv_bytes_per_row(wl):
    return 2 * wl.d * wl.elem_bytes             # one K row and one V row


def dense_bytes(wl, lens):
    n = sum(lens)
    return (n * wl.Hkv * kv_bytes_per_row(wl) + n * wl.Hq * 4 +
            wl.B * wl.Hq * wl.d * (wl.elem_bytes + 4) + wl.B * wl.Hq * 4)


def select_bytes(wl, lens):
    """HBM bytes the Selector of the fused slow step (sfi_slow_step) must move: the logits over J
    read once (its normaliser over J comes from the dense step), one 4-byte key written per
    (KV head, position of J) and read back by the candidate pass, and again by the emit when
    the chunked path ends in its resolve and emit passes rather than in the one-workgroup-per-
    unit finish (the library takes the finish when k_sel + max_len / 64 <= 16384), and the index
    rows written.  (Counting a second logit read and four passes over the keys gives an upper
    bound, for a Selector that computes its own normaliser.)  The candidates and kept
    entries, about 2 % of J, and the 16 KB histograms are not counted."""
    nJ = sum(max(0, n - wl.n_recent - wl.n_sink) for n in lens)
    key_passes = 2 if wl.k_sel + max(lens) // 64 <= 16384 else 3
    return wl.Hq * nJ * 4 + key_passes * wl.Hkv * nJ * 4 + sum(wl.Hkv * (wl.n_sink + wl.k_sel) * 4
                                                                for _ in lens)


def fast_bytes(wl, lens_t, n_idx_host, mask_host):
    tot = 0
    for b, N in enumerate(lens_t):
        rec = min(wl.n_recent, N)
        for h in range(wl.Hkv):
            if mask_host is not None and all(mask_host[b][h * wl.G:(h + 1) * wl.G]):
                continue
            rows = int(n_idx_host[b][h]) + rec
            tot += rows * kv_bytes_per_row(wl) + int(n_idx_host[b][h]) * 4
    return tot + wl.B * wl.Hq * wl.d * (wl.elem_bytes + 4) + wl.B * wl.Hq * 4


def counter_traffic(workload: str, key: str = "traffic_bytes_per_launch"):
    """HBM bytes from the committed rocprofv3 counter summary of this workload (FETCH_SIZE and
    WRITE_SIZE, each scaled by a known-size copy): per dense launch, or with key
    "fast_traffic_bytes_per_step" per fast step (partials kernel and combine).  None when there
    is none, or when the attention kernels or their launch plan (ATTN_SRCS) changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_counters.md")
    try:
        text = open(path).read()
        sha = attention_sources_sha256()
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith(key + "="):
            fields = dict(kv.split("=", 1) for kv in line.split())
            if fields.get("source_sha256") == sha:
                return int(fields[key])
    return None


def cpu_baseline(wl, layer, queries, lay0_host_lens, min_seconds=10.0, max_cycles=64):
    """The fp64 oracle on whole cycles of one layer (dense + select + mask + fast steps),
    repeated until at least min_seconds of CPU work have run; returns µs per decode step."""
    import oracle
    import numpy as np
    t_start = time.perf_counter()
    kw = {}
    if wl.paged:
        kw = dict(block_table=layer.block_table, block_size=wl.block_size,
                  max_blocks=layer.max_blocks)
    cache = oracle.Cache(layer.k, layer.v, layer.len0, wl.Hq, **kw)
    copy_s = time.perf_counter() - t_start
    parts = {"dense": 0.0, "select": 0.0, "mask": 0.0, "fast": 0.0}
    cycles = 0
    t_all = time.perf_counter()
    while cycles < max_cycles and (cycles == 0 or time.perf_counter() - t_all < min_seconds):
        t0 = time.perf_counter()
        eo, el, ez = oracle.dense(cache, queries[0])
        t1 = time.perf_counter()
        eidx, en, _ = oracle.select(lay0_host_lens, wl.Hq, wl.Hkv, ez, wl.n_sink, wl.n_recent,
                                    wl.k_sel)
        t2 = time.perf_counter()
        hm = oracle.sink_mask(ez[:, :, 0], el, wl.mask_frac) if wl.mask_frac > 0 else None
        t3 = time.perf_counter()
        for t in range(1, wl.cycle):
            oracle.sparse(cache.with_lens(np.asarray(lay0_host_lens) + t), queries[t], eidx, en,
                          wl.n_recent, hm)
        t4 = time.perf_counter()
        for k, v in (("dense", t1 - t0), ("select", t2 - t1), ("mask", t3 - t2), ("fast", t4 - t3)):
            parts[k] += v
        cycles += 1
    total = sum(parts.values())
    return {
        "value": round(total * 1e6 / (cycles * wl.cycle), 1),
        "unit": "us/step",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": (f"{cycles} whole cycles of one layer of {wl.name} (full batch {wl.B}, "
                   f"1 slow + {wl.cycle - 1} fast steps each), {total:.1f} s of oracle time: "
                   f"dense {parts['dense'] / cycles:.2f} s, select {parts['select'] / cycles:.3f} s, "
                   f"mask {parts['mask'] / cycles:.4f} s, fast steps {parts['fast'] / cycles:.2f} s "
                   f"per cycle; host copy of the cache ({copy_s:.1f} s) not timed"),
    }


def copy_calibration(mib: int, reps: int = 3):
    """A plain device copy of known size, for scaling the HBM byte counters (FETCH_SIZE,
    WRITE_SIZE) that rocprofv3 reports per dispatch: each dispatch reads and writes exactly
    mib MiB.  Runs after the timed region and is not part of any reported time."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"# copy calibration: {reps} copies of {mib} MiB", file=sys.stderr, flush=True)


def read_yardstick(B, torch, gib: int = 4, grids=(1024, 2048, 4096), reps: int = 10):
    """Achievable HBM read bandwidth on this machine: sfi_stream_read over a zeroed buffer of
    `gib` GiB (far beyond the 256 MB Infinity Cache), mean of `reps` event-timed launches for
    each grid size; the best grid is reported."""
    buf = torch.zeros(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    per_grid = {}
    for g in grids:
        for _ in range(2):
            B.sfi_stream_read(buf, g, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            B.sfi_stream_read(buf, g, sink)
        e1.record(stream)
        e1.synchronize()
        per_grid[g] = buf.numel() / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9
    del buf
    torch.cuda.empty_cache()
    best = max(per_grid, key=per_grid.get)
    return {"kernel": "sfi_stream_read (sequential 16-byte nontemporal loads)",
            "bytes": gib << 30, "workgroups": best, "gbps": round(per_grid[best], 1),
            "gbps_by_workgroups": {str(g): round(v, 1) for g, v in per_grid.items()}}


def group_dot_units(B, torch, wl, layers, queries, wg: int = 1024, reps: int = 3):
    """What the GQA group's dot products q_g . k_j cost on each arithmetic unit, next to the
    read they ride on (sfi_group_dot over every key row of a layer, in order, the workload's G
    heads of one query): no arithmetic, the vector ALUs, MFMA.  Each unit: two warm-up
    launches, then `reps` passes over the rotated layers (one launch per layer, so a launch
    does not find its rows in the Infinity Cache) timed with events; mean µs per launch.  Only
    for bf16 rows of 128 elements and G in 1, 2, 4, 8 (None otherwise)."""
    if wl.dtype != "bf16" or wl.d != 128 or wl.G not in (1, 2, 4, 8):
        return None
    stream = torch.cuda.current_stream()
    rows = []
    for lay in layers:
        flat = lay.k.reshape(-1)
        n = flat.numel() // 128 // 16 * 16
        rows.append(flat[: n * 128].view(n, 128))
    q = queries[0][0].reshape(-1, 128)[: wl.G].contiguous()
    part = torch.empty(wg, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    us, sums = {}, {}
    for unit in ("read", "valu", "mfma"):
        for r in rows[:2]:
            B.sfi_group_dot(r, q, unit, wg, part, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for r in rows:
                B.sfi_group_dot(r, q, unit, wg, part, sink)
        e1.record(stream)
        e1.synchronize()
        us[unit] = e0.elapsed_time(e1) * 1e3 / (reps * len(rows))
        if unit != "read":
            sums[unit] = float(part.double().sum())
    n_rows = rows[0].shape[0]
    return {"kernel": "sfi_group_dot (16-row groups of 4 KB per wavefront, 2 in flight)",
            "rows_per_launch": n_rows, "bytes_per_launch": n_rows * 256, "G": wl.G,
            "workgroups": wg, "read_us": round(us["read"], 2), "valu_us": round(us["valu"], 2),
            "mfma_us": round(us["mfma"], 2),
            "valu_over_read": round(us["valu"] / us["read"], 3),
            "mfma_over_read": round(us["mfma"] / us["read"], 3),
            "read_gbps": round(n_rows * 256 / (us["read"] * 1e-6) / 1e9, 1),
            "valu_mfma_sums_rel_diff": round(abs(sums["valu"] - sums["mfma"]) /
                                             max(1e-30, abs(sums["mfma"])), 8)}


def routed_fast_steps(B, torch, wl, descs, queries, logits, stride, idxs, nidxs, masks, ws,
                      idx_stride, L, gamma: float = 0.65):
    """Fast steps with inline group routing (sfi_sparse_decode_routed), each layer's slow-step
    lse as its cached normaliser: the slow step of every layer, then the cycle's fast steps in
    decode order (token by token, every layer in turn) timed as one block, twice.  Reports µs
    per fast step and the fraction of (sequence, KV head) groups bypassed."""
    dev = "cuda"
    stream = torch.cuda.current_stream()
    out = torch.empty((wl.B, wl.Hq, wl.d), device=dev)
    lse_f = torch.empty((wl.B, wl.Hq), device=dev)
    slow_lse = [torch.empty((wl.B, wl.Hq), device=dev) for _ in range(L)]
    routed = [torch.zeros((wl.B, wl.Hkv), dtype=torch.uint8, device=dev) for _ in range(L)]
    print("# routed fast steps", file=sys.stderr, flush=True)
    for li in range(L):
        d = descs[li]
        B.sfi_dense_decode(d[0], queries[li][0], out, slow_lse[li], logits[li], stride, ws)
        B.sfi_select(d[0], logits[li], stride, wl.n_sink, wl.n_recent, wl.k_sel, idxs[li],
                     idx_stride, nidxs[li], ws)
    times, frac = [], []
    for rep in range(2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(1, wl.cycle):
            for li in range(L):
                B.sfi_sparse_decode_routed(descs[li][t], queries[li][t], idxs[li], idx_stride,
                                           nidxs[li], wl.n_recent, masks[li], slow_lse[li],
                                           gamma, routed[li], out, lse_f, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / (L * (wl.cycle - 1)))
        frac += [float(r.float().mean()) for r in routed]
    return {"gamma": gamma, "fast_us": round(sum(times) / len(times), 2),
            "groups_routed_frac": round(sum(frac) / len(frac), 4),
            "normaliser": "lse of the slow step", "routing": "all heads of a KV group"}


def routed_sink_heavy(B, torch, synth, wl, layers, descs, stride, idx_stride, L, ws,
                      gamma: float = 0.65, extra: float = 2.1972245773362196):
    """The routed fast step at an operating point where most KV groups reach gamma: the sink
    recipe with token 0's key steadied (its part orthogonal to u scaled by 0.1, so its logit
    varies little between queries; restored afterwards) and its logit raised by ln 9 (token-0
    mass near 0.9), its own queries for every step, each layer's slow step (fused call) giving
    the index set and the cached normaliser.
    The same cycle's fast steps run in decode order once unrouted (sfi_sparse_decode) and once
    routed (sfi_sparse_decode_routed), each timed as one block, twice.  Bytes: the fast step's
    algorithmic bytes without and with the bypassed groups' rows and indices."""
    dev = "cuda"
    stream = torch.cuda.current_stream()
    print("# routed fast steps, sink-heavy queries", file=sys.stderr, flush=True)
    saved = [synth.steady_sink(lay, 0.1) for lay in layers]
    qs = [[synth.make_query(wl, li, t, device=dev, u=layers[li].u, sink_extra=extra)
           for t in range(wl.cycle)] for li in range(L)]
    out = torch.empty((wl.B, wl.Hq, wl.d), device=dev)
    lse_f = torch.empty((wl.B, wl.Hq), device=dev)
    slow_lse = [torch.empty((wl.B, wl.Hq), device=dev) for _ in range(L)]
    logits = torch.empty((wl.B, wl.Hq, stride), device=dev)
    idxs = [torch.empty((wl.B, wl.Hkv, idx_stride), dtype=torch.int32, device=dev) for _ in range(L)]
    nidxs = [torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device=dev) for _ in range(L)]
    routed = [torch.zeros((wl.B, wl.Hkv), dtype=torch.uint8, device=dev) for _ in range(L)]
    for li in range(L):
        B.sfi_slow_step(descs[li][0], qs[li][0], out, slow_lse[li], logits, stride, wl.n_sink,
                        wl.n_recent, wl.k_sel, idxs[li], idx_stride, nidxs[li], 0.0, None, ws)

    def block(route):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(1, wl.cycle):
            for li in range(L):
                if route:
                    B.sfi_sparse_decode_routed(descs[li][t], qs[li][t], idxs[li], idx_stride,
                                               nidxs[li], wl.n_recent, None, slow_lse[li], gamma,
                                               routed[li], out, lse_f, ws)
                else:
                    B.sfi_sparse_decode(descs[li][t], qs[li][t], idxs[li], idx_stride, nidxs[li],
                                        wl.n_recent, None, out, lse_f, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (L * (wl.cycle - 1))

    plain, rout, frac = [], [], []
    for rep in range(2):
        plain.append(block(False))
        rout.append(block(True))
        frac += [float(r.float().mean()) for r in routed]
    for lay, sv in zip(layers, saved):
        synth.restore_sink(lay, sv)
    lens0 = layers[0].len0_host
    n_idx_host = nidxs[0].cpu().tolist()
    mean = lambda x: sum(x) / len(x)
    full = mean([fast_bytes(wl, [n + t for n in lens0], n_idx_host, None)
                 for t in range(1, wl.cycle)])
    # the last step's decisions of layer 0, spread to its heads, as the bypassed groups' mask
    rmask = routed[0].repeat_interleave(wl.G, dim=1).cpu().tolist()
    kept = mean([fast_bytes(wl, [n + t for n in lens0], n_idx_host, rmask)
                 for t in range(1, wl.cycle)])
    return {"gamma": gamma, "token0_logit_raised_by": round(extra, 4),
            "token0_key_orthogonal_scale": 0.1,
            "groups_routed_frac": round(mean(frac), 4),
            "fast_us_unrouted": round(mean(plain), 2), "fast_us_routed": round(mean(rout), 2),
            "algorithmic_bytes_unrouted": int(full), "algorithmic_bytes_routed": int(kept),
            "normaliser": "lse of the slow step", "routing": "all heads of a KV group"}


def fast_floor(B, torch, wl, descs, idxs, nidxs, idx_stride, L, seq_bytes, grids=(256, 1024),
               seq_grids=(512, 1024)):
    """Floor of the fast step's access pattern: sfi_gather_read (the same rows, read once with
    no arithmetic, one launch) over the cycle's fast steps in decode order, timed as one block at
    each workgroup count, and the GPU-side cost of one launch with almost nothing to do (a 16 KB
    read by one workgroup, replayed from a captured graph).  The fast step itself needs two launches: its split-K
    partials and their merge.  Beside them, the size floor: sfi_stream_read of seq_bytes (the
    fast step's algorithmic bytes) from one of L buffers in turn, so that every read is as cold
    in the Infinity Cache as a fast step's rows, the best of seq_grids workgroup counts."""
    stream = torch.cuda.current_stream()
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    tiny = torch.zeros(4096, dtype=torch.int32, device="cuda")

    def block(fn):
        fn()
        torch.cuda.synchronize()
        best = None
        for rep in range(2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (L * (wl.cycle - 1))
            best = us if best is None else min(best, us)
        return best

    gather = {}
    for g in grids:
        gather[g] = block(lambda: [B.sfi_gather_read(descs[li][t], idxs[li], idx_stride,
                                                     nidxs[li], wl.n_recent, g, sink)
                                   for t in range(1, wl.cycle) for li in range(L)])
    # one launch with almost nothing to do, replayed from a captured graph so that the host's
    # own call overhead (larger than the GPU's per-launch cost) does not set the pace
    n_launch = L * (wl.cycle - 1)
    launch = graph_replay(torch, lambda: [B.sfi_stream_read(tiny, 1, sink) for _ in range(n_launch)],
                          n_launch)
    best = min(gather, key=gather.get)
    n = int(seq_bytes) // 4096 * 4096
    bufs = [torch.zeros(n, dtype=torch.uint8, device="cuda") for _ in range(L)]
    seq = {}
    for g in seq_grids:
        seq[g] = block(lambda: [B.sfi_stream_read(bufs[li], g, sink)
                                for t in range(1, wl.cycle) for li in range(L)])
    del bufs
    torch.cuda.empty_cache()
    sbest = min(seq, key=seq.get)
    return {"gather_read_us": round(gather[best], 2), "gather_read_workgroups": best,
            "gather_read_us_by_workgroups": {str(g): round(v, 2) for g, v in gather.items()},
            "one_launch_us": round(launch, 2),
            "two_launch_floor_us": round(gather[best] + launch, 2),
            "sequential_read_same_bytes_us": round(seq[sbest], 2),
            "sequential_read_workgroups": sbest}


def graph_replay(torch, run, per_replay: int, reps: int = 3):
    """The stack cycle run() captured once in a HIP graph (torch.cuda.CUDAGraph: the library's
    calls queue kernels only) and replayed back to back, timed on the host clock like the
    eager timed region.  Returns µs per decode step of one layer (per_replay steps a replay)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / (reps * per_replay)
    del g
    return round(us, 3)


def retention_sweep(B, torch, synth, ratios=(0.016, 0.031, 0.0625, 0.125, 0.25, 0.5, 1.0),
                    n_sets=16, rounds=3):
    """Dense against sparse attention on one layer shaped like the SFI page's retention table
    (Sec. 5: KV 16K, batch 16; here 32/8 heads, d 128, bf16, sink 4 + recent 256), with the
    selected positions drawn as sentence-like spans.  retention = |I| / N, the attended
    positions over the context.  Each ratio rotates over n_sets different selections so the
    rows a call reads were not left in the 256 MB Infinity Cache by the previous calls."""
    import dataclasses
    dev = "cuda"
    wl = synth.Workload("retention_16k_b16", 6000, 16, 32, 8, 128, "bf16", 16384, 4, 256, 0, 2)
    lay = synth.make_layer(wl, 0, device=dev)
    N = wl.n0
    lens = lay.len_at(0).to(dev)
    desc = B.KVDesc(lay.k, lay.v, lens, N, wl.Hq)
    q = synth.make_query(wl, 0, 0, device=dev)
    stride = (N + 3) // 4 * 4
    logits = torch.empty((wl.B, wl.Hq, stride), device=dev)
    out = torch.empty((wl.B, wl.Hq, wl.d), device=dev)
    lse = torch.empty((wl.B, wl.Hq), device=dev)
    J_lo, J_hi = wl.n_sink, N - wl.n_recent
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    ws = B.workspace(desc, idx_stride=N, n_recent=wl.n_recent, device=dev)
    dense_us = timed(lambda i: B.sfi_dense_decode(desc, q, out, lse, logits, stride, ws), 10)
    nolog_us = timed(lambda i: B.sfi_dense_decode(desc, q, out, lse, None, stride, ws), 10)
    rows = []
    for r in ratios:
        k = min(J_hi - J_lo, max(0, int(round(r * N)) - wl.n_sink - wl.n_recent))
        stride_i = wl.n_sink + max(k, 1)
        sets = []
        for s in range(n_sets):
            g = torch.Generator().manual_seed(7000 + s)
            idx = torch.zeros((wl.B, wl.Hkv, stride_i), dtype=torch.int32)
            for b in range(wl.B):
                for h in range(wl.Hkv):
                    sel = synth.span_selection(J_lo, J_hi, k, g) if k > 0 else torch.zeros(0, dtype=torch.int32)
                    row = torch.cat([torch.arange(wl.n_sink, dtype=torch.int32), sel])
                    idx[b, h, :row.numel()] = row
            n_idx = torch.full((wl.B, wl.Hkv), wl.n_sink + k, dtype=torch.int32)
            sets.append((idx.to(dev), n_idx.to(dev)))
        wsr = B.workspace(desc, idx_stride=stride_i, n_recent=wl.n_recent, device=dev)
        sparse_us = timed(lambda i: B.sfi_sparse_decode(desc, q, sets[i % n_sets][0], stride_i,
                                                        sets[i % n_sets][1], wl.n_recent, None,
                                                        out, lse, wsr), rounds * n_sets)
        slots = wl.n_sink + k + wl.n_recent
        rows.append({"retention": round(slots / N, 4), "k_sel": k, "sparse_us": round(sparse_us, 2),
                     "dense_over_sparse": round(dense_us / sparse_us, 2),
                     "dense_nolog_over_sparse": round(nolog_us / sparse_us, 2)})
        del sets, wsr
    return {"shape": "B 16, 32/8 heads, d 128, bf16, N 16384, sink 4, recent 256, spans",
            "dense_us": round(dense_us, 2), "dense_nolog_us": round(nolog_us, 2), "rows": rows}


def context_sweep(B, torch, synth, contexts=(32768, 65536, 131072, 262144, 524288), L=4,
                  reps=3):
    """Dense step, Selector and fast step of one Llama-3.1-8B-shaped layer (batch 1, 32/8
    heads, d 128, bf16, sink 4 + recent 256 + k 2048) over contexts of 32K to 512K, each call
    timed over L rotated layers (fast steps in decode order) so no layer's rows are re-read from
    the Infinity Cache.  fast_us is the fast-step block replayed from a captured graph,
    fast_eager_us the same block launched from Python, which the host paces at this size."""
    dev = "cuda"
    ev = lambda: torch.cuda.Event(enable_timing=True)
    rows = []
    for N in contexts:
        wl = synth.Workload(f"ctx_{N}", 8000 + N // 1024, 1, 32, 8, 128, "bf16", N, 4, 256, 2048, 16)
        lays = [synth.make_layer(wl, li, device=dev) for li in range(L)]
        T = wl.cycle
        lens = [lays[0].len_at(t).to(dev) for t in range(T)]
        descs = [[B.KVDesc(lay.k, lay.v, lens[t], lay.max_len_at(t), wl.Hq) for t in range(T)]
                 for lay in lays]
        qs = [[synth.make_query(wl, li, t, device=dev) for t in range(T)] for li in range(L)]
        stride = (N + 3) // 4 * 4
        istride = wl.n_sink + wl.k_sel
        logits = [torch.empty((1, wl.Hq, stride), device=dev) for _ in range(L)]
        idx = [torch.empty((1, wl.Hkv, istride), dtype=torch.int32, device=dev) for _ in range(L)]
        nidx = [torch.empty((1, wl.Hkv), dtype=torch.int32, device=dev) for _ in range(L)]
        out = torch.empty((1, wl.Hq, wl.d), device=dev)
        lse = torch.empty((1, wl.Hq), device=dev)
        ws = B.workspace(descs[0][T - 1], idx_stride=istride, n_recent=wl.n_recent, device=dev)

        def dense(with_logits):
            for li in range(L):
                B.sfi_dense_decode(descs[li][0], qs[li][0], out, lse,
                                   logits[li] if with_logits else None, stride, ws)

        def select():
            for li in range(L):
                B.sfi_select(descs[li][0], logits[li], stride, wl.n_sink, wl.n_recent, wl.k_sel,
                             idx[li], istride, nidx[li], ws)

        def fast():
            for t in range(1, T):
                for li in range(L):
                    B.sfi_sparse_decode(descs[li][t], qs[li][t], idx[li], istride, nidx[li],
                                        wl.n_recent, None, out, lse, ws)

        def timed(fn, per):
            fn()
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return 1e3 * e0.elapsed_time(e1) / (reps * per)

        d_us = timed(lambda: dense(True), L)
        n_us = timed(lambda: dense(False), L)
        s_us = timed(select, L)
        # back-to-back fast steps of a small layer outrun the host's launches from Python, so
        # the block is also replayed from a captured graph (the GPU's own time)
        fe_us = timed(fast, L * (T - 1))
        f_us = graph_replay(torch, fast, L * (T - 1))
        d_bytes = dense_bytes(wl, [N])
        f_bytes = fast_bytes(wl, [N + 1], nidx[0].cpu().tolist(), None)
        rows.append({"context": N, "dense_us": round(d_us, 1), "dense_nolog_us": round(n_us, 1),
                     "dense_gbps": round(d_bytes / (d_us * 1e-6) / 1e9, 1),
                     "select_us": round(s_us, 1), "fast_us": round(f_us, 2),
                     "fast_eager_us": round(fe_us, 2),
                     "fast_gbps": round(f_bytes / (f_us * 1e-6) / 1e9, 1),
                     "value_us": round((d_us + s_us + (T - 1) * f_us) / T, 2)})
        print(f"#   context {N}: {rows[-1]}", file=sys.stderr, flush=True)
        del lays, descs, qs, logits, idx, nidx, ws
        torch.cuda.empty_cache()
    return {"shape": "B 1, 32/8 heads, d 128, bf16, sink 4, recent 256, k 2048, cycle 16, "
                     f"{L} rotated layers", "rows": rows}


def synthetic_selection_fast_steps(B, torch, synth, wl, layers, descs, queries, out, lse, ws,
                                   idx_stride, L):
    """Fast steps on the workload's synthetic selections instead of the Selector's: sentence-
    like spans of 10-40 positions, and uniformly scattered positions (the two variants the
    ragged workload is stated with), each timed over the fast steps of a whole cycle of every
    rotated layer in decode order."""
    dev = "cuda"
    res = {}
    for kind in ("spans", "scattered"):
        sets = []
        for li in range(L):
            i, n = synth.synthetic_index_set(layers[li], kind, seed=900 + li, idx_stride=idx_stride)
            sets.append((i.to(dev), n.to(dev)))

        def run():
            for t in range(1, wl.cycle):
                for li in range(L):
                    B.sfi_sparse_decode(descs[li][t], queries[li][t], sets[li][0], idx_stride,
                                        sets[li][1], wl.n_recent, None, out, lse, ws)
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        res[kind + "_us"] = round(1e3 * e0.elapsed_time(e1) / (L * (wl.cycle - 1)), 2)
    return res


def key_norms(torch, wl, lay, n: int, stride: int):
    """fp32 [B][Hkv][stride] norms of the cached keys at positions < n (the statistics the
    full Selector's prior reads; computed once per layer with torch, outside any timing)."""
    out = torch.ones((wl.B, wl.Hkv, stride), dtype=torch.float32, device=lay.k.device)
    if not wl.paged:
        for b in range(wl.B):
            out[b, :, :n] = torch.linalg.vector_norm(lay.k[b, :, :n], dim=-1, dtype=torch.float32)
        return out
    phys = torch.linalg.vector_norm(lay.k, dim=-1, dtype=torch.float32)   # [n_blk][Hkv][bs]
    pos = torch.arange(n, device=lay.k.device)
    for b in range(wl.B):
        blk = lay.block_table[b, pos // wl.block_size].long()
        out[b, :, :n] = phys[blk, :, pos % wl.block_size].transpose(0, 1)
    return out


def refined_selector(B, torch, wl, layers, descs, logits, stride, idx_stride, L, reps=3):
    """sfi_select_refined (prior, fusion, Soft-NMS, cross-head exclusivity) on every rotated
    layer's slow-step logits, timed as a block beside the plain Selector."""
    dev = "cuda"
    n = layers[0].max_len_at(0)
    norms = [key_norms(torch, wl, layers[li], n, stride) for li in range(L)]
    ws = B.workspace(descs[0][0], idx_stride=idx_stride, n_recent=wl.n_recent, device=dev,
                     refined=True)
    idx = torch.empty((wl.B, wl.Hkv, idx_stride), dtype=torch.int32, device=dev)
    n_idx = torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device=dev)
    params = dict(B.REFINE_DEFAULTS)

    def refined():
        for li in range(L):
            B.sfi_select_refined(descs[li][0], logits[li], stride, norms[li], stride, wl.n_sink,
                                 wl.n_recent, wl.k_sel, params, idx, idx_stride, n_idx, ws)

    def plain():
        for li in range(L):
            B.sfi_select(descs[li][0], logits[li], stride, wl.n_sink, wl.n_recent, wl.k_sel, idx,
                         idx_stride, n_idx, ws)

    res = {}
    for name, fn in (("select_refined_us", refined), ("select_plain_us", plain)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(1e3 * e0.elapsed_time(e1) / (reps * L), 2)
    del norms, ws
    res["params"] = {k.rstrip("_"): round(v, 4) for k, v in params.items()}
    return res


def two_segment_steps(B, torch, wl, descs, queries, idxs, nidxs, masks, out, lse, ws,
                      idx_stride, L):
    """The two-segment layout: sfi_reorg of every rotated layer's selection (once per cycle),
    then the cycle's fast steps on the compact segment (sfi_sparse_decode_compact) in decode
    order (token by token, every layer in turn), timed as blocks beside the same fast steps
    gathered from the cache."""
    dev = "cuda"
    segs = []
    for li in range(L):
        ck = torch.empty((wl.B, wl.Hkv, idx_stride, wl.d), dtype=wl.torch_dtype, device=dev)
        segs.append((ck, torch.empty_like(ck),
                     torch.empty((wl.B, wl.Hkv, idx_stride), dtype=torch.int32, device=dev)))

    def reorg():
        for li in range(L):
            B.sfi_reorg(descs[li][0], idxs[li], idx_stride, nidxs[li], *segs[li])

    def compact():
        for t in range(1, wl.cycle):
            for li in range(L):
                B.sfi_sparse_decode_compact(descs[li][t], queries[li][t], *segs[li], idx_stride,
                                            nidxs[li], wl.n_recent, masks[li], out, lse, ws)

    def gather():
        for t in range(1, wl.cycle):
            for li in range(L):
                B.sfi_sparse_decode(descs[li][t], queries[li][t], idxs[li], idx_stride,
                                    nidxs[li], wl.n_recent, masks[li], out, lse, ws)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / reps

    reorg_us = timed(reorg) / L
    compact_us = timed(compact) / (L * (wl.cycle - 1))
    gather_us = timed(gather) / (L * (wl.cycle - 1))
    n_sel = sum(int(x) for x in nidxs[0].flatten().tolist())
    row = wl.d * wl.elem_bytes
    units = wl.B * wl.Hkv
    reorg_bytes = n_sel * 2 * row + units * idx_stride * 2 * row + n_sel * 4 + units * idx_stride * 4
    del segs
    return {"reorg_us": round(reorg_us, 2),
            "reorg_gbps": round(reorg_bytes / (reorg_us * 1e-6) / 1e9, 1),
            "reorg_bytes": int(reorg_bytes),
            "fast_us": round(compact_us, 2), "gather_fast_us": round(gather_us, 2),
            "fast_saving_per_cycle_us": round((gather_us - compact_us) * (wl.cycle - 1), 2)}


def layered_slow_step(B, torch, wl, descs, queries, logits, stride, idxs, nidxs, masks, ws,
                      idx_stride, slots: int = 4, reps: int = 5):
    """The slow step over every rotated layer: sfi_slow_step layer after layer, against
    sfi_slow_step_layers (the same kernels, the Selector and mask of each layer on a second
    stream, a ring of `slots` logits buffers and Selector workspaces).  Host clock around whole
    slow steps."""
    L = len(descs)
    R = min(slots, L)
    dev = "cuda"
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    d0 = [descs[li][0] for li in range(L)]
    outs = [torch.empty((wl.B, wl.Hq, wl.d), device=dev) for _ in range(L)]
    lses = [torch.empty((wl.B, wl.Hq), device=dev) for _ in range(L)]
    sel_ws = [ws] + [torch.empty_like(ws) for _ in range(R - 1)]
    dense_ws = torch.empty_like(ws)
    events = [torch.cuda.Event() for _ in range(R)]
    attn_ev, done_ev = torch.cuda.Event(), torch.cuda.Event()
    has_mask = masks[0] is not None

    def sequential():
        for l in range(L):
            s = l % R
            B.sfi_slow_step(d0[l], queries[l][0], outs[l], lses[l], logits[s], stride, wl.n_sink,
                            wl.n_recent, wl.k_sel, idxs[l], idx_stride, nidxs[l], wl.mask_frac,
                            masks[l] if has_mask else None, sel_ws[s])

    def pipelined():
        B.sfi_slow_step_layers(d0, [queries[l][0] for l in range(L)], outs, lses, logits[:R],
                               stride, sel_ws, dense_ws, wl.n_sink, wl.n_recent, wl.k_sel, idxs,
                               idx_stride, nidxs, wl.mask_frac, masks if has_mask else None,
                               stream, side, events, attn_ev, done_ev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / reps

    print("# layered slow step", file=sys.stderr, flush=True)
    t_seq = timed(sequential)
    t_pipe = timed(pipelined)
    return {"layers": L, "slots": R, "sequential_us": round(t_seq, 1),
            "pipelined_us": round(t_pipe, 1), "per_layer_sequential_us": round(t_seq / L, 2),
            "per_layer_pipelined_us": round(t_pipe / L, 2)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the decode-attention path runs on a single MI355X "
              f"and has no multi-GPU mode (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_kv_attention_dense_amd import binding as B
    from sparse_kv_attention_dense_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"
    wl = synth.WORKLOADS[args.workload]
    L = max(1, args.layers)
    print(f"# building {L} layers of {wl.name}", file=sys.stderr, flush=True)

    layers, descs, queries, logits, idxs, nidxs, masks, outs, lses = [], [], [], [], [], [], [], [], []
    lens_t = None
    for li in range(L):
        lay = synth.make_layer(wl, li, device=dev)
        layers.append(lay)
        if lens_t is None:
            lens_t = [lay.len_at(t).to(dev) for t in range(wl.cycle)]
            max_t = [lay.max_len_at(t) for t in range(wl.cycle)]
        kw = dict(block_table=lay.block_table, block_size=wl.block_size) if wl.paged else {}
        descs.append([B.KVDesc(lay.k, lay.v, lens_t[t], max_t[t], wl.Hq, **kw)
                      for t in range(wl.cycle)])
        queries.append([synth.make_query(wl, li, t, device=dev, u=lay.u) for t in range(wl.cycle)])
        stride = (max_t[0] + 3) // 4 * 4
        logits.append(torch.empty((wl.B, wl.Hq, stride), device=dev))
        idxs.append(torch.empty((wl.B, wl.Hkv, wl.n_sink + wl.k_sel), dtype=torch.int32, device=dev))
        nidxs.append(torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device=dev))
        masks.append(torch.zeros((wl.B, wl.Hq), dtype=torch.uint8, device=dev)
                     if wl.mask_frac > 0 else None)
        print(f"#   layer {li} ready", file=sys.stderr, flush=True)
    stride = logits[0].shape[-1]
    out = torch.empty((wl.B, wl.Hq, wl.d), device=dev)
    lse = torch.empty((wl.B, wl.Hq), device=dev)
    idx_stride = wl.n_sink + wl.k_sel
    ws = B.workspace(descs[0][wl.cycle - 1], idx_stride=idx_stride, n_recent=wl.n_recent, device=dev)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def cycle(rec):
        """One slow-fast cycle of the L-layer stack in decode order: token 0 runs the slow step
        of every layer in turn (dense with logits, Selector, mask), then each later token runs
        the fast step of every layer in turn.  Between two fast steps of one layer the other
        layers' steps run, as when a decode step passes through a model's layers, so a layer's
        selected rows are not still in the 256 MB Infinity Cache from its previous step.
        rec = "none": no events; "dense": events around each dense call only (the timed
        region); "all": events around each slow-step call and around the block of fast steps."""
        marks = []
        for li in range(L):
            d0 = descs[li]
            e = [ev() for _ in range(3)] if rec != "none" else None
            # the slow step in one call: dense with logits, Selector (its normaliser over J from
            # the dense kernels), mask; e[0] and e[1] are recorded by the library right before
            # and after the dense kernels, so host-side checks are never inside the interval
            B.sfi_slow_step(d0[0], queries[li][0], out, lse, logits[li], stride, wl.n_sink,
                            wl.n_recent, wl.k_sel, idxs[li], idx_stride, nidxs[li],
                            wl.mask_frac, masks[li], ws, dense_done=e[1] if e else None,
                            dense_begin=e[0] if e else None)
            if rec == "all":
                e[2].record(stream)
            marks.append(e)
        fe = [ev(), ev()] if rec == "all" else None
        if fe:
            fe[0].record(stream)
        for t in range(1, wl.cycle):
            for li in range(L):
                B.sfi_sparse_decode(descs[li][t], queries[li][t], idxs[li], idx_stride,
                                    nidxs[li], wl.n_recent, masks[li], out, lse, ws)
        if fe:
            fe[1].record(stream)
        return marks, fe

    print("# warmup", file=sys.stderr, flush=True)
    for s in range(args.warmup):
        cycle("none")
    torch.cuda.synchronize()
    # Timed region: whole stack cycles back to back; the only events are the two around each
    # dense call (the roofline kernel), so the wall clock is not inflated by event records.
    print("# timed region", file=sys.stderr, flush=True)
    evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        evs.append(cycle("dense"))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    mean = lambda x: sum(x) / len(x)
    dense_us = 1e3 * mean([e[0].elapsed_time(e[1]) for marks, _ in evs for e in marks])
    # Breakdown: separate stack cycles with events around the Selector, the mask and the block
    # of fast steps (each event pair adds a few µs of its own, so the breakdown is not used for
    # value; the fast steps are timed as one block and divided by their number).
    print("# breakdown", file=sys.stderr, flush=True)
    evs = [cycle("all") for s in range(max(1, min(args.steps, 2)))]
    torch.cuda.synchronize()
    # Selector and (when the workload has one) mask: from the library's event after the dense
    # kernels to the end of the slow-step call
    select_us = 1e3 * mean([e[1].elapsed_time(e[2]) for marks, _ in evs for e in marks])
    fast_us = 1e3 * mean([fe[0].elapsed_time(fe[1]) / (L * (wl.cycle - 1)) for _, fe in evs])

    # Spread: one more stack cycle in decode order with events around every single call
    # (p10 / p50 / p90), and the dense step without its logit write as a reference for the
    # cost of the logits.
    dense_calls, nolog_calls, fast_calls, sep_calls, mask_calls = [], [], [], [], []
    if not args.no_spread:
        print("# per-call spread", file=sys.stderr, flush=True)
        pairs = {"dense": [], "nolog": [], "fast": [], "select_sep": [], "mask": []}

        def timed_call(kind, fn):
            e = (ev(), ev())
            e[0].record(stream)
            fn()
            e[1].record(stream)
            pairs[kind].append(e)

        # the separate calls of the slow step, each timed on its own: the dense step, the
        # Selector with its own log-sum-exp pass (sfi_select), the mask
        for li in range(L):
            d0 = descs[li]
            timed_call("dense", lambda: B.sfi_dense_decode(d0[0], queries[li][0], out, lse,
                                                           logits[li], stride, ws))
            timed_call("select_sep", lambda: B.sfi_select(d0[0], logits[li], stride, wl.n_sink,
                                                          wl.n_recent, wl.k_sel, idxs[li],
                                                          idx_stride, nidxs[li], ws))
            if masks[li] is not None:
                timed_call("mask", lambda: B.sfi_sink_bypass_mask(d0[0], logits[li], stride, lse,
                                                                  wl.mask_frac, masks[li]))
        for t in range(1, wl.cycle):
            for li in range(L):
                timed_call("fast", lambda: B.sfi_sparse_decode(
                    descs[li][t], queries[li][t], idxs[li], idx_stride, nidxs[li], wl.n_recent,
                    masks[li], out, lse, ws))
        for li in range(L):
            timed_call("nolog", lambda: B.sfi_dense_decode(descs[li][0], queries[li][0], out,
                                                           lse, None, stride, ws))
        torch.cuda.synchronize()
        dense_calls = [1e3 * a.elapsed_time(b) for a, b in pairs["dense"]]
        nolog_calls = [1e3 * a.elapsed_time(b) for a, b in pairs["nolog"]]
        fast_calls = [1e3 * a.elapsed_time(b) for a, b in pairs["fast"]]
        sep_calls = [1e3 * a.elapsed_time(b) for a, b in pairs["select_sep"]]
        mask_calls = [1e3 * a.elapsed_time(b) for a, b in pairs["mask"]]

    def pct(xs):
        if not xs:
            return None
        xs = sorted(xs)
        at = lambda q: xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]
        return [round(at(0.1), 2), round(at(0.5), 2), round(at(0.9), 2)]

    graph_us = None
    if not args.no_graph:
        print("# stack cycle replayed from a HIP graph", file=sys.stderr, flush=True)
        graph_us = graph_replay(torch, lambda: cycle("none"), wl.cycle * L)


    print("# fast steps on synthetic selections", file=sys.stderr, flush=True)
    synth_fast = synthetic_selection_fast_steps(B, torch, synth, wl, layers, descs, queries, out,
                                                lse, ws, idx_stride, L)

    routed = routed_heavy = None
    if wl.sink and not args.no_routed:
        routed = routed_fast_steps(B, torch, wl, descs, queries, logits, stride, idxs, nidxs,
                                   masks, ws, idx_stride, L)
        routed_heavy = routed_sink_heavy(B, torch, synth, wl, layers, descs, stride, idx_stride,
                                         L, ws)

    layered = None
    if L >= 2 and not args.no_layered:
        layered = layered_slow_step(B, torch, wl, descs, queries, logits, stride, idxs, nidxs,
                                    masks, ws, idx_stride)

    refined = None
    if not args.no_refined:
        print("# full Selector", file=sys.stderr, flush=True)
        refined = refined_selector(B, torch, wl, layers, descs, logits, stride, idx_stride, L)

    two_seg = None
    if not args.no_two_segment:
        print("# two-segment layout", file=sys.stderr, flush=True)
        two_seg = two_segment_steps(B, torch, wl, descs, queries, idxs, nidxs, masks, out, lse,
                                    ws, idx_stride, L)

    print("# streaming-read yardstick", file=sys.stderr, flush=True)
    yard = read_yardstick(B, torch)
    print("# group dot products by arithmetic unit", file=sys.stderr, flush=True)
    gdot = group_dot_units(B, torch, wl, layers, queries)

    lens0 = layers[0].len0_host
    n_idx_host = nidxs[0].cpu().tolist()
    mask_host = masks[0].cpu().tolist() if masks[0] is not None else None
    d_bytes = dense_bytes(wl, lens0)
    s_bytes = select_bytes(wl, lens0)
    f_bytes = mean([fast_bytes(wl, [n + t for n in lens0], n_idx_host, mask_host)
                    for t in range(1, wl.cycle)])
    f_bytes_unmasked = mean([fast_bytes(wl, [n + t for n in lens0], n_idx_host, None)
                             for t in range(1, wl.cycle)])
    dense_gbps = d_bytes / (dense_us * 1e-6) / 1e9
    fast_gbps = f_bytes / (fast_us * 1e-6) / 1e9
    select_gbps = s_bytes / (select_us * 1e-6) / 1e9
    value = ms_per_step * 1e3 / (wl.cycle * L)
    traffic = counter_traffic(wl.name)

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_cycle": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.d, "context": wl.n0, "n_sink": wl.n_sink,
                   "n_recent": wl.n_recent, "k_sel": wl.k_sel, "cycle": wl.cycle,
                   "mask_frac": wl.mask_frac, "layers_rotated": L,
                   "step": f"{L} layers x (1 slow (dense+select{'+mask' if wl.mask_frac else ''}) + "
                           f"{wl.cycle - 1} fast), token-major"},
        "slow_us": round(dense_us + select_us, 2),
        "fast_us": round(fast_us, 2),
        "dense_us": round(dense_us, 2),
        "select_us": round(select_us, 2),
        "mask_us": round(mean(mask_calls), 2) if mask_calls else 0.0,
        "select_separate_us": round(mean(sep_calls), 2) if sep_calls else None,
        "dense_gbps": round(dense_gbps, 1),
        "fast_gbps": round(fast_gbps, 1),
        "select_gbps": round(select_gbps, 1),
        "fast_pct_peak": round(100 * fast_gbps / PEAK_HBM_GBS, 1),
        "dense_nolog_us": round(mean(nolog_calls), 2) if nolog_calls else None,
        "spread_us": {"p10_p50_p90": True, "dense": pct(dense_calls),
                      "dense_nolog": pct(nolog_calls), "fast": pct(fast_calls),
                      "calls": {"dense": len(dense_calls), "fast": len(fast_calls)}},
        "tokens_per_s": round(wl.B * 1e6 / value, 1),
        "steps_explained": "value is us per decode step of one layer (amortised over the cycle); "
                           "ms_per_step = ms_per_cycle is one timed bench step: a whole stack "
                           f"cycle of {L} layers x {wl.cycle} decode steps",
        "hbm_frac_by_step": {"dense": round(dense_gbps / PEAK_HBM_GBS, 4),
                             "selector": round(select_gbps / PEAK_HBM_GBS, 4),
                             "fast": round(fast_gbps / PEAK_HBM_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(dense_gbps, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(dense_gbps / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": "sfi_dense_decode (attention_kernel)",
                     "algorithmic_bytes": d_bytes},
        "fast_roofline": {"bound": "hbm", "achieved": round(fast_gbps, 1), "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(fast_gbps / PEAK_HBM_GBS, 4),
                          "traffic": counter_traffic(wl.name, "fast_traffic_bytes_per_step"),
                          "algorithmic_bytes": int(f_bytes),
                          "bytes_saved_by_masked_groups": int(f_bytes_unmasked - f_bytes)},
    }
    result["read_yardstick"] = yard
    if gdot is not None:
        result["group_dot"] = gdot
    if graph_us is not None:
        result["graph_cycle"] = {"us_per_step": graph_us, "eager_us_per_step": round(value, 3),
                                 "what": "the same stack cycle captured once in a HIP graph "
                                         "and replayed (no host launch cost)"}
    if refined is not None:
        refined["value_if_used_us"] = round(
            (dense_us + refined["select_refined_us"] + (mean(mask_calls) if mask_calls else 0.0)
             + (wl.cycle - 1) * fast_us)
            / wl.cycle, 3)
        result["select_refined"] = refined
    if two_seg is not None:
        two_seg["value_if_used_us"] = round(
            (dense_us + select_us + two_seg["reorg_us"] +
             (wl.cycle - 1) * two_seg["fast_us"]) / wl.cycle, 3)
        result["two_segment"] = two_seg
    result["roofline"]["frac_of_measured_read"] = round(dense_gbps / yard["gbps"], 4)
    result["fast_roofline"]["frac_of_measured_read"] = round(fast_gbps / yard["gbps"], 4)
    print("# fast-step floor (gather read, one launch, sequential read)", file=sys.stderr,
          flush=True)
    floor = fast_floor(B, torch, wl, descs, idxs, nidxs, idx_stride, L, f_bytes)
    floor["sequential_read_frac_of_peak"] = round(
        f_bytes / (floor["sequential_read_same_bytes_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    floor["gather_read_frac_of_peak"] = round(f_bytes / (floor["gather_read_us"] * 1e-6) / 1e9
                                              / PEAK_HBM_GBS, 4)
    floor["two_launch_floor_frac_of_peak"] = round(
        f_bytes / (floor["two_launch_floor_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    floor["fast_us_over_two_launch_floor"] = round(fast_us / floor["two_launch_floor_us"], 3)
    result["fast_roofline"]["floor"] = floor
    result["fast_synthetic_selections"] = synth_fast
    if routed is not None:
        result["routed_fast"] = routed
    if routed_heavy is not None:
        result["routed_fast_sink_heavy"] = routed_heavy
    if layered is not None:
        result["slow_step_layers"] = layered
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
    if not args.no_cpu_baseline:
        print("# cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        host_q = [q.cpu() for q in queries[0]]
        result["cpu_baseline"] = cpu_baseline(wl, layers[0], host_q, lens0)
    if args.retention_sweep or args.context_sweep:
        del layers, descs, queries, logits, idxs, nidxs, masks
        torch.cuda.empty_cache()
    if args.retention_sweep:
        print("# retention sweep", file=sys.stderr, flush=True)
        result["retention_sweep"] = retention_sweep(B, torch, synth)
    if args.context_sweep:
        print("# context sweep", file=sys.stderr, flush=True)
        result["context_sweep"] = context_sweep(B, torch, synth)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
