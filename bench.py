"""Benchmark of the CSA2 read path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_256k]

A step is one pass of the whole layer stack of the workload over its batch: for
decode_256k, 32 queries each over its own 262,144-entry cache through Full (indexer over
the whole context, Top-512, HSI pool of 2,048 blocks, attention), Reindex (indexer over
the pool, Top-512, attention) and three Reuse layers (attention). The step's kernels are
captured once into a HIP graph and replayed; W untimed replays, then K timed replays
bracketed by device synchronisation. Before the W warm-up replays the step is replayed for
--settle-ms (default 300 ms) so that the GPU's clocks have settled as in continuous
serving; a short warm-up alone leaves the first timed steps a few percent slow. Inputs are
seeded synthetic tensors already resident in HBM. Prints one JSON line.

roofline: the dominant kernel is the Full-layer indexer, launched as the step launches it.
Queries that share one sequence (prefill_128k_m2, encoder_128k_m2) read each key row once
per group of queries, so there the indexer is priced against the bf16 matrix peak
(8,192 flops per (query, entry) pair) instead of HBM.
Its algorithmic bytes per launch are 128 B of indexer K read + 0.5 B of block maximum
written per (query, entry) pair (+ 4 B of score where the step keeps the scores: stacks
without a pool; + 0.5 B of block statistics where the decoder Full layer's one-kernel
selection reads them), plus the indexer queries and weights; its average launch duration is
measured with HIP events on its own stream over K back-to-back launches.

roofline.traffic: HBM bytes per indexer launch from rocprofv3 counters (FETCH_SIZE and
WRITE_SIZE, each divided by what the same counter reports per byte for a plain 1 GiB copy
kernel), read from the committed counter summary; null when the indexer source has changed
since the counters were taken. `--profile-kernel` runs only the indexer and the copy, for
those counter runs.

--coarse hisa swaps the HSI pool for the block-mean two-stage filter in every indexer layer
(block means resident, as a decoder keeps them up to date); the dominant kernel is then the
block-mean scorer (256 B of bf16 mean key read + 4 B of score written per (query, block)).
needle_recall (decode workloads, which plant positions): the share of planted positions in
the Full layer's Top-K, the pool and the Reindex layer's Top-K; for the second needle set
(planted along the Reindex layer's own indexer query) the share the pool keeps, the share
the Reindex Top-K keeps and the share lost outside the pool; --recall adds the same under
the block-mean filter.

Workloads whose caches total less than 512 MiB (decode_32k, tiny_decode_4k) would otherwise
be timed out of the 256 MiB last-level cache: their caches are copied until the copies
exceed 512 MiB (at most 8) and consecutive steps read consecutive copies.

cpu_baseline: the fp64 oracle (oracle/) run on the host over a bounded sample of the same
workload's queries (whole layer stack per query), scaled to queries/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 matrix peak
PEAK_FP8_TFLOPS = 5000.0      # dense fp8 matrix peak (the MXFP8-query indexer)
FLOPS_PER_PAIR = 32 * 128 * 2   # indexer multiply-adds of one (query, entry) pair
INDEXER_SRC = os.path.join(ROOT, "compressed_kv_cache_csa2_amd", "csrc", "index_score.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "index_score_full_decode_256k.md")
COPY_BYTES = 1 << 30
ROTATE_BYTES = 512 << 20      # a workload whose caches are smaller is timed over rotated copies


def source_sha256(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload):
    """HBM bytes per Full-indexer launch from the committed counter summary, if it was taken
    on this workload with the current indexer source; else None."""
    if workload != "decode_256k" or not os.path.exists(TRAFFIC_SUMMARY):
        return None
    fields = {}
    for line in open(TRAFFIC_SUMMARY):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    try:
        if fields.get("indexer source sha256") != source_sha256(INDEXER_SRC):
            return None
        return float(fields["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def full_indexer(wl, buf, C, stream=None):
    """The Full-layer indexer as the step launches it: block maxima only in a pooled stack
    (with the block statistics where the one-kernel selection follows), over the workload's
    key format."""
    from compressed_kv_cache_csa2_amd import layers
    lay = next(l for l in wl.layers if l.mode == "full")
    layers.index_score(wl, C.FULL, lay, None if wl.with_pool else buf.scores,
                       buf.block_max, ld_scores=buf.scores.shape[1], stream=stream, buf=buf,
                       block_aux=buf.block_aux if layers.fused_full_select(wl) else None)


def rotated_copies(wl):
    """The workload, plus copies of its caches (same values) when they total less than
    ROTATE_BYTES, so that consecutive steps do not find their rows in cache."""
    import dataclasses
    import math
    tensors = [wl.k_cache, wl.kv_fp4, wl.kv_scale, wl.k_codes, wl.k_scales]
    size = sum(t.numel() * t.element_size() for t in tensors if t is not None)
    if size >= ROTATE_BYTES or wl.group_caches:
        return [wl]
    n = min(8, math.ceil(ROTATE_BYTES / max(1, size)))
    cl = lambda t: None if t is None else t.clone()
    return [wl] + [dataclasses.replace(wl, k_cache=cl(wl.k_cache), kv_fp4=cl(wl.kv_fp4),
                                       kv_scale=cl(wl.kv_scale), k_codes=cl(wl.k_codes),
                                       k_scales=cl(wl.k_scales)) for _ in range(n - 1)]


def hisa_stage1(wl, buf, C, means, stream=None):
    """First stage of the block-mean filter for the first indexer layer."""
    lay = wl.layers[0]
    C.csa2_index_score_bf16(C.FULL, lay.q_idx, lay.w, means.km, means.km_start, means.n_blocks,
                            buf.block_max, stream=stream)


def hisa_stage1_bytes(wl):
    import torch
    blocks = int(((wl.n_visible.to(torch.int64) + 7) // 8).sum())
    return blocks * (256 + 4) + wl.n_q * (32 * 128 * 2 + 32 * 4)


def _recall(planted, nv, pool=None, idx=None):
    """Share of the planted positions inside a pool (block ids) or an index set."""
    import torch
    hit = total = 0
    for t in range(planted.shape[0]):
        p = torch.unique(planted[t][planted[t] < nv[t]])
        total += p.numel()
        if pool is not None:
            hit += int(torch.isin(p // 8, pool[t]).sum())
        else:
            hit += int(torch.isin(p, idx[t].to(torch.int64)).sum())
    return hit / max(1, total)


def needle_recall(wl, buf, C, means=None):
    """Share of the planted positions kept by each selection of the stack: the Full layer's
    Top-K, the pool, and the Reindex layer's Top-K (which uses its own query, unrelated to
    the Full-layer planting). Decoder stacks also carry needles planted along the Reindex
    layer's own indexer query: "reindex_needles" gives the share of those whose block the
    pool keeps (with HSI, the Full layer's pool; with the block-mean filter, the Reindex
    layer's own), the share its Top-K keeps, and the share lost because the block lies
    outside the pool (a later indexer cannot recover it). With block means, the same under
    the block-mean filter, whose every indexer layer builds its own pool (the first layer's
    pool is taken on its own)."""
    import torch
    from compressed_kv_cache_csa2_amd import layers
    planted = wl.planted.cpu()
    planted_re = None if wl.planted_re is None else wl.planted_re.cpu()
    nv = wl.n_visible.cpu()
    li_full = next(i for i, l in enumerate(wl.layers) if l.mode == "full")
    li_re = next((i for i, l in enumerate(wl.layers) if l.mode == "reindex"), None)

    def count(pl):
        return int(sum(torch.unique(pl[t][pl[t] < nv[t]]).numel() for t in range(pl.shape[0])))

    out = {}
    for coarse in (("hsi", "hisa") if means is not None else ("hsi",)):
        res = {}
        if coarse == "hisa":
            layers.hisa_select(wl, wl.layers[li_full], buf, means, buf.idx[li_full])
            torch.cuda.synchronize()
            res["full_topk"] = _recall(planted, nv, idx=buf.idx[li_full].cpu())
            res["pool"] = _recall(planted, nv, pool=buf.pool.cpu())
        layers.run_layers(wl, buf, coarse=coarse, means=means)
        torch.cuda.synchronize()
        if coarse == "hsi":
            res["full_topk"] = _recall(planted, nv, idx=buf.idx[li_full].cpu())
            if wl.with_pool:
                res["pool"] = _recall(planted, nv, pool=buf.pool.cpu())
        if li_re is not None:
            res["reindex_topk"] = _recall(planted, nv, idx=buf.idx[li_re].cpu())
        res["needles"] = count(planted)
        if planted_re is not None and li_re is not None and wl.with_pool:
            # after the pass, buf.pool is the pool the Reindex layer selected from
            in_pool = _recall(planted_re, nv, pool=buf.pool.cpu())
            res["reindex_needles"] = {
                "pool": in_pool,
                "reindex_topk": _recall(planted_re, nv, idx=buf.idx[li_re].cpu()),
                "lost_outside_pool": 1.0 - in_pool,
                "needles": count(planted_re),
            }
        out[coarse] = res
    return out


def q8_selection_overlap(wl, buf):
    """For a workload whose indexer query is quantised to MXFP8: the mean overlap of each
    selection of the stack with the one the bf16 query makes on the same data (both run
    through the library): the Full layer's Top-K, the pool (decoder stacks) and the Reindex
    layer's Top-K."""
    import torch
    from compressed_kv_cache_csa2_amd import layers
    li_full = next((i for i, l in enumerate(wl.layers) if l.mode == "full"), None)
    li_re = next((i for i, l in enumerate(wl.layers) if l.mode == "reindex"), None)
    if li_full is None:
        return None
    layers.run_layers(wl, buf)
    ref = layers.alloc_buffers(wl)
    wl.q8 = False
    try:
        layers.run_layers(wl, ref)
    finally:
        wl.q8 = True
    torch.cuda.synchronize()

    def mean_overlap(a, b):
        a, b = a.cpu(), b.cpu()
        tot = 0.0
        for t in range(a.shape[0]):
            x, y = a[t][a[t] >= 0], b[t][b[t] >= 0]
            tot += int(torch.isin(x, y).sum()) / max(1, y.numel())
        return tot / max(1, a.shape[0])

    out = {"full_topk": mean_overlap(buf.idx[li_full], ref.idx[li_full])}
    if wl.with_pool:
        out["pool"] = mean_overlap(buf.pool, ref.pool)
    if li_re is not None:
        out["reindex_topk"] = mean_overlap(buf.idx[li_re], ref.idx[li_re])
    return out


def profile_kernels(wl, buf, C, launches, means=None):
    """Only the dominant kernel (the Full-layer indexer, or the block-mean scorer when
    `means` is given) and a plain copy of COPY_BYTES, for counter collection."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(launches):
        if means is not None:
            hisa_stage1(wl, buf, C, means)
        else:
            full_indexer(wl, buf, C)
        torch.neg(src, out=dst)   # reads and writes COPY_BYTES each
    torch.cuda.synchronize()
    print(f"[bench] profile launches done: {launches} x (indexer, copy of {COPY_BYTES} B)",
          file=sys.stderr, flush=True)


def algorithmic_bytes(wl, k=512, coarse="hsi"):
    """Bytes the method must move per step: every visible indexer-K row of a Full layer,
    the pool's rows of a Reindex layer, and per attention layer the selected FP4 rows
    (288 B), the 128 FP8 window rows (512 B), the 64x512 bf16 query and output. Under the
    block-mean filter every indexer layer reads its blocks' bf16 mean keys (256 B per 8
    positions) and the pool's rows."""
    import torch
    nv = wl.n_visible.to(torch.int64).cpu()
    total = 0
    for lay in wl.layers:
        if coarse == "hisa" and lay.mode in ("full", "reindex"):
            total += int(((nv + 7) // 8).sum()) * 256
            total += int(torch.clamp(nv, max=16384).sum()) * key_bytes(wl)
        elif lay.mode == "full" and wl.shared_start is not None:
            total += wl.n_ctx * key_bytes(wl)      # one sequence: each key row once
        elif lay.mode == "full":
            total += int(nv.sum()) * key_bytes(wl)
        elif lay.mode == "reindex":
            total += int(torch.clamp(nv, max=16384).sum()) * key_bytes(wl)
        sel = torch.clamp(nv, max=k) if lay.mode != "swa" else torch.zeros_like(nv)
        total += int(sel.sum()) * 288 + wl.n_q * (128 * 512 + 2 * 64 * 512 * 2)
    return total


def key_bytes(wl):
    """Bytes of one indexer-key row: 128 (E4M3) or 64 + 4 (MXFP4)."""
    return 68 if wl.k_codes is not None else 128


def indexer_bytes_per_launch(wl):
    import torch
    from compressed_kv_cache_csa2_amd import layers
    pairs = int(wl.n_visible.to(torch.int64).sum())
    # Per pair: the key row read, 4 B of score where the row is kept, 0.5 B of block
    # maximum, and 0.5 B of block statistics where the one-kernel selection reads them.
    written = 0.5 if wl.with_pool else 4 + 0.5
    if layers.fused_full_select(wl):
        written += 0.5
    return pairs * (key_bytes(wl) + written) + wl.n_q * (32 * 128 * 2 + 32 * 4)


def cpu_baseline(wl, target_s, max_q):
    """Time the oracle stack on queries 0, 1, ... until target_s seconds have passed."""
    import numpy as np

    import oracle.csa2_oracle as O
    from compressed_kv_cache_csa2_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    done = 0
    t_total = 0.0
    # Queries are taken in order and cycled until target_s seconds of oracle time (the copy
    # of each query's inputs to the host is outside the timed region).
    while done < max_q and t_total < target_s:
        seq = synth.sequence_to_host(wl, done % wl.n_q)
        t0 = time.perf_counter()
        nv = seq["n_visible"]
        idx = pool = None
        for lay in seq["layers"]:
            keys = seq["k_codes"] if "k_codes" in seq else lay["k_cache"]
            if lay["mode"] == "full":
                r = O.full_layer(lay["q_idx"], lay["w"], keys, 0, nv, lay["q"], lay["kv_fp4"],
                                 lay["kv_scale"], lay["window_kv"], 0, lay["n_swa"],
                                 wl.softmax_scale, with_pool=wl.with_pool,
                                 k_scales=seq.get("k_scales"))
                pool = r.get("pool")
            elif lay["mode"] == "reindex":
                r = O.reindex_layer(lay["q_idx"], lay["w"], keys, 0, nv, pool, lay["q"],
                                    lay["kv_fp4"], lay["kv_scale"], lay["window_kv"], 0,
                                    lay["n_swa"], wl.softmax_scale, k_scales=seq.get("k_scales"))
            elif lay["mode"] == "swa":
                r = O.swa_layer(lay["q"], lay["window_kv"], 0, lay["n_swa"], wl.softmax_scale)
            else:
                r = O.reuse_layer(idx, lay["q"], lay["kv_fp4"], lay["kv_scale"], 0,
                                  lay["window_kv"], 0, lay["n_swa"], wl.softmax_scale)
            if lay["mode"] != "swa":
                idx = r["idx"]
        t_total += time.perf_counter() - t0
        done += 1
        np.asarray(r["out"]).sum()
    note = (" with the bf16 indexer query (the oracle's MXFP8-query scorers are not timed)"
            if wl.q8 else "")
    return {"value": done / t_total, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "threads": "BLAS threads of the numpy oracle (threadpoolctl)",
            "host": host_cpu(),
            "sample": f"{done} query stacks of {wl.name} (its {wl.n_q} queries taken in order, "
                      f"cycled), whole layer stack per query{note}, {t_total:.1f} s of oracle "
                      "time"}


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo), its logical CPU count and the CPUs this
    process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count()
    return {"model": model, "logical_cpus": os.cpu_count(), "allowed_cpus": allowed}


def kernel_label(wl, hisa):
    """Name of the dominant kernel as the step launches it."""
    if hisa:
        return "index_score_kernel (block-mean scorer, bf16 mean keys)"
    keys = "MXFP4 keys" if wl.k_codes is not None else "E4M3 keys"
    if wl.shared_start is not None:
        name = ("index_score_shared_q8_kernel (grouped Full indexer, " if wl.q8 else
                "index_score_shared2_kernel (grouped Full indexer, ") + keys
    elif wl.q8:
        name = "index_score_q8_kernel (Full-layer indexer, " + keys + ", MXFP8 query"
    elif wl.k_codes is not None:
        name = "index_score_full_wide_fp4_kernel (Full-layer indexer, " + keys
    else:
        name = "index_score_full_e4m3_kernel (Full-layer indexer, " + keys
    from compressed_kv_cache_csa2_amd import layers
    if layers.fused_full_select(wl):
        return name + ", block maxima and block statistics)"
    return name + (", block maxima only)" if wl.with_pool else ")")


def measure(name, args, C, layers, synth, with_breakdown=False, with_recall=False):
    """One workload: the step timed as a replayed HIP graph and the dominant kernel timed
    back to back, both with HIP events on the step's stream. Returns the figures and the
    workload."""
    import torch
    t0 = time.time()
    wl = synth.make_workload(name, device="cuda:0")
    torch.cuda.synchronize()
    print(f"[bench] {name}: generated in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    buf = layers.alloc_buffers(wl)
    hisa = args.coarse == "hisa"
    means = None
    if hisa or with_recall:
        if not wl.with_pool or wl.k_codes is not None:
            print("--coarse hisa / --recall need a pooled decoder workload with E4M3 keys",
                  file=sys.stderr)
            sys.exit(2)
        means = layers.build_block_means(wl)
        torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    copies = rotated_copies(wl)
    turn = [0]

    def step(w):
        layers.run_layers(w, buf, stream=stream, coarse=args.coarse, means=means)

    with torch.cuda.stream(stream):
        for w in copies:
            step(w)
    torch.cuda.synchronize()

    if not args.no_graph:
        graphs = []
        for w in copies:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(w)
            graphs.append(g)
        torch.cuda.synchronize()

        def run():
            graphs[turn[0] % len(graphs)].replay()
            turn[0] += 1
    else:
        def run():
            step(copies[turn[0] % len(copies)])
            turn[0] += 1

    # Clock settle: replay the step for about --settle-ms before the warm-up steps, so that
    # the timed steps see the steady clocks of a GPU that is already serving.
    t_settle = time.perf_counter()
    with torch.cuda.stream(stream):
        while time.perf_counter() - t_settle < args.settle_ms * 1e-3:
            for _ in range(20):
                run()
            stream.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            run()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(args.steps):
            run()
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] {name}: timed {args.steps} steps: {ms_step * 1e3:.1f} us/step (host wall "
          f"{wall / args.steps * 1e6:.1f} us/step)", file=sys.stderr, flush=True)

    # Dominant kernel: the Full-layer indexer (or the block-mean scorer), launched back to
    # back on `stream`.
    def dominant():
        if hisa:
            hisa_stage1(wl, buf, C, means, stream=stream)
        else:
            full_indexer(copies[turn[0] % len(copies)], buf, C, stream=stream)
            turn[0] += 1

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        dominant()
        e0.record(stream)
        for _ in range(args.steps):
            dominant()
        e1.record(stream)
    torch.cuda.synchronize()
    idx_us = e0.elapsed_time(e1) * 1e3 / args.steps
    idx_bytes = hisa_stage1_bytes(wl) if hisa else indexer_bytes_per_launch(wl)
    achieved = idx_bytes / (idx_us * 1e-6) / 1e9

    if with_breakdown:
        breakdown(wl, buf, C, layers, stream, hisa, means)
    recall = needle_recall(wl, buf, C, means if with_recall else None) \
        if wl.planted is not None else None
    q8_overlap = q8_selection_overlap(wl, buf) if wl.q8 and not hisa else None
    step_bytes = algorithmic_bytes(wl, coarse=args.coarse)
    res = {
        "workload": wl.name, "wl": wl, "copies": len(copies), "ms_step": ms_step,
        "value": wl.n_q / (ms_step * 1e-3),
        "step_bytes": step_bytes,
        "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": None if hisa else measured_traffic(wl.name),
                     "kernel": kernel_label(wl, hisa), "launch_us": idx_us,
                     "bytes_per_launch": idx_bytes},
        "recall": recall,
        "q8_overlap": q8_overlap,
    }
    if wl.shared_start is not None:
        pairs = int(wl.n_visible.to(torch.int64).sum())
        tflops = pairs * FLOPS_PER_PAIR / (idx_us * 1e-6) / 1e12
        peak = PEAK_FP8_TFLOPS if wl.q8 else PEAK_BF16_TFLOPS
        res["roofline"].update({"bound": "mfma", "achieved": tflops, "peak": peak,
                                "unit": "TFLOP/s", "frac": tflops / peak,
                                "flops_per_launch": pairs * FLOPS_PER_PAIR})
        del res["roofline"]["bytes_per_launch"]
    return res


def breakdown(wl, buf, C, layers, stream, hisa, means):
    """Per-call event timings of one eager pass of the stack, to stderr."""
    import torch
    fused = layers.fused_full_select(wl)   # the Full layer's selection is one kernel
    names = []
    evs = []
    with torch.cuda.stream(stream):
        for li, lay in enumerate(wl.layers):
            for part in ("score", "pool", "rescore", "topk", "attn"):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                if hisa and lay.mode in ("full", "reindex") and part != "attn":
                    if part == "score":
                        C.csa2_index_score_bf16(C.FULL, lay.q_idx, lay.w, means.km,
                                                means.km_start, means.n_blocks,
                                                buf.block_max, stream=stream)
                    elif part == "pool":
                        C.csa2_block_pool(buf.block_max, wl.n_visible, buf.pool,
                                          stream=stream)
                    elif part == "rescore":
                        layers.index_score(wl, C.REINDEX, lay, buf.re_scores,
                                           pool_blocks=buf.pool, stream=stream, buf=buf)
                    else:
                        C.csa2_topk(buf.re_scores, buf.idx[li], pool_blocks=buf.pool,
                                    stream=stream)
                elif part == "score" and lay.mode == "full":
                    full_indexer(wl, buf, C, stream=stream)
                elif (part in ("rescore", "topk") and lay.mode == "full" and wl.with_pool
                      and fused):
                    continue
                elif part == "pool" and lay.mode == "full" and wl.with_pool and fused:
                    layers.full_select(wl, lay, buf, buf.idx[li], stream=stream)
                elif part == "rescore" and lay.mode == "full" and wl.with_pool:
                    layers.index_score(wl, C.REINDEX, lay, buf.re_scores,
                                       pool_blocks=buf.cand, stream=stream, buf=buf)
                elif part == "score" and lay.mode == "reindex":
                    layers.index_score(wl, C.REINDEX, lay, buf.re_scores,
                                       pool_blocks=buf.pool, stream=stream, buf=buf)
                elif part == "topk" and lay.mode == "full" and wl.with_pool:
                    C.csa2_topk(buf.re_scores, buf.idx[li], pool_blocks=buf.cand,
                                stream=stream)
                elif part == "topk" and lay.mode == "full":
                    C.csa2_topk(buf.scores, buf.idx[li], n_valid=wl.n_visible,
                                block_max=buf.block_max, stream=stream)
                elif part == "topk" and lay.mode == "reindex":
                    C.csa2_topk(buf.re_scores, buf.idx[li], pool_blocks=buf.pool, stream=stream)
                elif part == "pool" and lay.mode == "full" and wl.with_pool:
                    C.csa2_pool_candidates(buf.block_max, wl.n_visible, buf.pool, buf.cand,
                                           stream=stream)
                elif part == "attn":
                    _, kv_fp4, kv_scale = wl.cache(lay.group)
                    C.csa2_sparse_attn(lay.q, kv_fp4, kv_scale, wl.kv_start,
                                       buf.published[li], lay.window_kv, lay.swa_start,
                                       lay.n_swa, wl.softmax_scale, buf.out[li], buf.lse[li],
                                       buf.workspace, stream=stream)
                else:
                    continue
                b.record(stream)
                names.append(f"L{li}:{lay.mode}:{part}")
                evs.append((a, b))
    torch.cuda.synchronize()
    for n, (a, b) in zip(names, evs):
        print(f"[bench] {n:24s} {a.elapsed_time(b) * 1e3:9.1f} us", file=sys.stderr)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # A step is ~0.4 ms: 50 warm-up steps let clocks and caches settle, 200 timed steps
    # take under 0.1 s.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode_256k")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="replay the step this long before the warm-up steps (clock settle)")
    ap.add_argument("--no-1m", action="store_true",
                    help="skip the decode_1m sub-record of the default decode_256k run")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--breakdown", action="store_true", help="per-call timings to stderr")
    ap.add_argument("--coarse", choices=("hsi", "hisa"), default="hsi",
                    help="coarse filter of the indexer layers (pooled stacks)")
    ap.add_argument("--recall", action="store_true",
                    help="also report needle recall under the block-mean filter")
    ap.add_argument("--profile-kernel", type=int, default=0, metavar="N",
                    help="only launch the Full indexer and a 1 GiB copy N times (counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the decode batch "
              "shards by sequence with no exchange, so one GPU's throughput is the figure; see "
              "the design notes for the multi-GPU layout.", file=sys.stderr)
        sys.exit(2)

    import torch

    from compressed_kv_cache_csa2_amd import csa2 as C
    from compressed_kv_cache_csa2_amd import layers, synth

    torch.cuda.set_device(0)
    if args.profile_kernel:
        wl = synth.make_workload(args.workload, device="cuda:0")
        buf = layers.alloc_buffers(wl)
        means = layers.build_block_means(wl) if args.coarse == "hisa" else None
        torch.cuda.synchronize()
        profile_kernels(wl, buf, C, args.profile_kernel, means)
        return
    head = measure(args.workload, args, C, layers, synth, with_breakdown=args.breakdown,
                   with_recall=args.recall)
    wl = head["wl"]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds, 100000)
    line = {
        "metric": "decode queries/sec + achieved HBM GB/s (% of peak)",
        "value": head["value"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if wl.q8 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "queries": wl.n_q, "context_entries": wl.n_ctx,
                   "layers": [l.mode for l in wl.layers], "index_topk": 512,
                   "sliding_window": 128, "pool_blocks": 2048 if wl.with_pool else 0,
                   "indexer_keys": "mxfp4" if wl.k_codes is not None else "e4m3",
                   "indexer_query": "mxfp8" if wl.q8 else "bf16",
                   "coarse_filter": args.coarse, "rotated_copies": head["copies"],
                   "launch": "eager" if args.no_graph else "hip_graph"},
        "step_hbm_gbps": head["step_hbm_gbps"],
        "step_hbm_frac": head["step_hbm_gbps"] / PEAK_HBM_GBPS,
        "step_algorithmic_bytes": head["step_bytes"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
    }
    if head["recall"] is not None:
        line["needle_recall"] = head["recall"]
    if head["q8_overlap"] is not None:
        line["q8_selection_overlap"] = head["q8_overlap"]
    if args.workload == "decode_256k" and args.coarse == "hsi" and not args.no_1m:
        # The metric's 1M half: the same measurement of decode_1m (64 queries of 1,048,576
        # entries each) in the same run, on the same GPU.
        del head, wl
        torch.cuda.empty_cache()
        sub = measure("decode_1m", args, C, layers, synth)
        line["decode_1m"] = {
            "value": sub["value"], "unit": "queries/s", "ms_per_step": sub["ms_step"],
            "queries": sub["wl"].n_q, "context_entries": sub["wl"].n_ctx,
            "step_hbm_gbps": sub["step_hbm_gbps"],
            "step_hbm_frac": sub["step_hbm_gbps"] / PEAK_HBM_GBPS,
            "step_algorithmic_bytes": sub["step_bytes"],
            "roofline": sub["roofline"],
            "needle_recall": sub["recall"],
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
