"""Benchmark of head-aware SegPaged attention on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config I]   (default I = 2)

One step = one segpaged_attention call (the persistent prefill or decode kernel plus the
fixed-order combine) over the workload's batch, with the layout already built and the work
list planned (page "RedKnot SegPagedAttention runtime design", section 5: layout work happens
once at KV-write time; rebuilding it per call was a slowdown). The build is timed once,
separately. The same run times this library's dense-plus-mask path on the same inputs and the
fp64 CPU oracle on a bounded sample of rows, and checks the sampled rows against the oracle.

Prints one JSON line. FLOPs count visible (query, key) pairs only, 4*D per pair; bytes count
the stored K/V rows once plus Q, O and the page tables.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (matrix and vector)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
EVENT_EVERY = 4             # main-kernel events on every 4th timed step
BUILD_RUNS = 5              # the build's time is the median of this many rebuilds


def head_window(kind: int, window: int, L: int) -> int:
    """LOCAL window of a head for a request of context length L (kind 2: L // divisor)."""
    return max(1, L // window) if kind == 2 else window


def retrieval_kept(S: int, permille: int, L: int, nq: int) -> int:
    """Prefix tokens a RETRIEVAL head keeps (its sink and the top fraction of the rest)."""
    prefix = max(0, L - nq)
    s = min(S, prefix)
    return s + -(-permille * (prefix - s) // 1000)


def visible_counts(case) -> np.ndarray:
    """Visible (query, key) pairs per (request, KV head), one query head's worth."""
    out = np.zeros((case.B, case.Hkv), dtype=np.float64)
    for b in range(case.B):
        L, nq = int(case.ctx_len[b]), int(case.q_len[b])
        p = np.arange(L - nq, L, dtype=np.int64)
        for h in range(case.Hkv):
            kind, S, W = (int(x) for x in case.policy[h])
            W = head_window(kind, W, L)
            if kind == 0:
                n = p + 1
            elif kind == 3:
                n = retrieval_kept(S, W, L, nq) + (p - (L - nq) + 1)
            else:
                lo = np.maximum(0, p - W + 1)
                n = (p - lo + 1) + np.minimum(S, lo)
            out[b, h] = float(n.sum())
    return out


def stored_rows(case, kv_len) -> float:
    return float(np.asarray(kv_len, dtype=np.float64).sum())


def source_hash() -> str:
    """Hash of the library sources with comments and blank space removed (a kernel change,
    not a comment edit, invalidates stored counter results)."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "head_aware_paged_segpaged_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_oracle_sample(case, budget_rows: int, importance=None, budget_s: float = 0.0):
    """Times the fp64 oracle on a bounded sample of (request, query head) rows: at most
    budget_rows rows, and with budget_s > 0 it stops after the (request, query head) that takes
    the time past budget_s."""
    import oracle

    rng = np.random.default_rng(1234)
    picks = []
    for b in range(case.B):
        nq = int(case.q_len[b])
        if nq == 0:
            continue
        for hq in range(case.Hq):
            picks.append((b, hq, nq))
    rng.shuffle(picks)
    per = max(1, budget_rows // max(1, len(picks)))
    sample = []
    rows = 0
    for b, hq, nq in picks:
        if rows >= budget_rows:
            break
        toks = np.arange(nq) if nq <= per else np.sort(rng.choice(nq, per, replace=False))
        sample.append((b, hq, toks))
        rows += len(toks)
    t0 = time.perf_counter()
    outs = []
    for b, hq, toks in sample:
        outs.append(oracle.attention_rows(case.q, case.k, case.v, case.ctx_len, case.q_len,
                                          case.policy, case.Hq, case.Hkv, case.scale, case.dtype,
                                          b, hq, toks, importance=importance))
        if budget_s > 0 and time.perf_counter() - t0 > budget_s:
            break
    secs = time.perf_counter() - t0
    sample = sample[:len(outs)]
    rows = sum(len(t) for _, _, t in sample)
    # visible pairs of the sample
    G = case.Hq // case.Hkv
    pairs = 0.0
    for b, hq, toks in sample:
        L, nq = int(case.ctx_len[b]), int(case.q_len[b])
        p = L - nq + toks
        kind, S, W = (int(x) for x in case.policy[hq // G])
        W = head_window(kind, W, L)
        if kind == 0:
            pairs += float((p + 1).sum())
        elif kind == 3:
            pairs += float((retrieval_kept(S, W, L, nq) + (p - (L - nq) + 1)).sum())
        else:
            lo = np.maximum(0, p - W + 1)
            pairs += float(((p - lo + 1) + np.minimum(S, lo)).sum())
    return sample, outs, secs, pairs, rows


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2,
                    help="workload index (0-7; 5 = the 32K-128K slice of the decode workload, "
                         "6 = the decode workload with context-adaptive LOCAL windows, "
                         "7 = the decode workload with two RETRIEVAL heads); default 2, the "
                         "Llama-3.3-70B-shaped layer (batch 4, 2048-token chunks of 16K-32K "
                         "contexts), the largest workload that runs on one GPU")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="rows of the CPU-oracle sample (default: up to 64K rows spread over every "
                         "(request, query head), stopping once about 15 s of oracle work is done)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense+mask timing")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra steps, each after reading a 512 MiB scratch buffer (evicts "
                         "the L2s and the MALL), whose main-kernel median is reported as "
                         "cold_cache; 0 skips them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB device-to-device 3 times (a plain copy "
                         "kernel of known size for calibrating rocprofv3 byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn two rocprofv3 --pmc runs of this workload "
                         "(FETCH_SIZE, then WRITE_SIZE, each with --copy-calibration) into "
                         "HBM bytes per launch of its main kernel in profiles/traffic.json")
    ap.add_argument("--counters-from", nargs="+", metavar="PMC_DIR",
                    help="no GPU run: average every counter of these rocprofv3 --pmc run "
                         "directories over the dispatches of this workload's main kernel and "
                         "store them in profiles/counters.json (with the MFMA busy share, the "
                         "bf16 MFMA FLOPs per dispatch against the visible-pair FLOPs, and the "
                         "per-wave instruction counts per KV step)")
    ap.add_argument("--counters-kernel", choices=("main", "build"), default="main",
                    help="with --counters-from: the kernel whose dispatches are averaged (the "
                         "workload's main attention kernel, or the build's scatter kernel)")
    ap.add_argument("--build-layers", type=int, default=0, metavar="N",
                    help="also time one build of N layers of this workload's shape into one "
                         "shared page pool (layer l's KV-head policies are the workload's "
                         "rolled by l heads); reported as build_layers; 0 skips it")
    ap.add_argument("--decode-steps", type=int, default=0, metavar="N",
                    help="decode workloads: also time N decode steps over a growable layout, "
                         "each appending every request's new token (segpaged_append) and then "
                         "attending (segpaged_decode); reported as decode_append; 0 skips it")
    ap.add_argument("--decode-graph", action="store_true",
                    help="with --decode-steps: also time the steps as replays of one captured "
                         "HIP graph (append + decode), inputs copied into its buffers per step")
    ap.add_argument("--decode-requests", type=int, default=0, metavar="R",
                    help="with --decode-steps: only the workload's first R requests (a small "
                         "decode batch, where launch costs matter); 0 = all")
    ap.add_argument("--page-order", choices=("shuffled", "sequential"), default="shuffled",
                    help="order of the free list the build hands pages out from: a seeded "
                         "permutation of the pool (default: pages scattered over the pool, as "
                         "after allocator churn) or 0, 1, 2, ... (each segment's pages adjacent)")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time torch's bf16 GEMM (hipBLASLt) at 4096^3..16384^3: what a "
                         "vendor-tuned dense contraction reaches on this GPU, for context")
    args = ap.parse_args()
    if args.traffic_from:
        return write_traffic(args)
    if args.counters_from:
        return write_counters(args)
    if args.gemm_reference:
        return gemm_reference()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch

    from head_aware_paged_segpaged_amd import (DenseMaskLayer, HipEvent, SegPagedDecoder,
                                               SegPagedLayer, SegPagedLayers)
    from workloads import config_case, decode_tokens, importance_scores
    from workloads import free_list as shuffled_free_list

    def free_list(seed, n):
        if args.page_order == "sequential":
            return np.arange(n, dtype=np.int32)
        return shuffled_free_list(seed, n)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    case = config_case(args.config)
    t_gen = time.perf_counter() - t_gen
    print("workload %s generated in %.1f s" % (case.name, t_gen), file=sys.stderr, flush=True)

    def up(x):
        if case.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v = up(case.q), up(case.k), up(case.v)
    layer = SegPagedLayer(case.dtype, case.Hq, case.Hkv, case.D, case.P, case.ctx_len, case.q_len,
                          case.policy, dev)
    fl = free_list(case.seed, layer.n_virt)
    stream = torch.cuda.current_stream()

    # Build: allocated once, then timed separately, with cold caches, as the median of a few
    # rebuilds into the same buffers: the library call (host checks, table upload, scatter
    # kernels) on wall clock, and on HIP events around it on the stream.
    # RETRIEVAL heads keep the top fraction of their prefix by a seeded importance input
    importance = importance_scores(case) if (case.policy[:, 0] == 3).any() else None
    # the library takes importance head-major ([Hkv][T]); the oracle reads it token-major
    layer.build(k, v, fl, importance=None if importance is None else
                np.ascontiguousarray(importance.T))
    # Cache eviction between timed runs: READ a 512 MiB buffer that is never written. A
    # written buffer would leave dirty lines in the L2s and the MALL whose write-back then
    # lands inside the timed kernel (measured: a plain read kernel loses 11 % that way).
    scratch = torch.empty(64 << 20, dtype=torch.int64, device=dev)

    def evict():
        scratch.sum()

    walls, streams = [], []
    for _ in range(BUILD_RUNS):
        evict()
        torch.cuda.synchronize()
        b0, b1 = HipEvent(), HipEvent()
        t0 = time.perf_counter()
        b0.record(stream)
        layer.rebuild(k, v, fl)
        b1.record(stream)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        streams.append(b0.elapsed_ms(b1))
    build_s, build_ms = float(np.median(walls)), float(np.median(streams))
    kv_len = layer.kv_len.cpu().numpy()
    elem = 2 if case.dtype == "bf16" else 4
    rows = stored_rows(case, kv_len)
    build_bytes = 2.0 * 2.0 * rows * case.D * elem  # read + write, K and V

    layer.plan()
    scale = case.scale
    out = torch.empty_like(q)

    # Warmup, then K timed steps bracketed by synchronisation; HIP events around the whole
    # region, and around the main (attention) kernel of every EVENT_EVERY-th step (each pair of
    # event records adds a few microseconds to its step, which matters for the short workloads;
    # a uniform sample of the timed steps keeps that out of the step time).
    sampled = list(range(0, args.steps, EVENT_EVERY))
    ev_m = {i: (HipEvent(), HipEvent()) for i in sampled}
    for _ in range(args.warmup):
        layer.attention(q, scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = HipEvent(), HipEvent()
    e0.record(stream)
    for i in range(args.steps):
        layer.attention(q, scale, out=out, events=ev_m.get(i))
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_ms(e1)
    ms_step = total_ms / args.steps
    main_ms = float(np.mean([a.elapsed_ms(b) for a, b in ev_m.values()]))
    err = layer.check()
    assert err == 0, "device-side error %d" % err

    pairs = visible_counts(case).sum() * (case.Hq // case.Hkv)
    flops = 4.0 * case.D * pairs
    io_bytes = (2.0 * rows * case.D * elem                      # stored K and V rows
                + 2.0 * case.tq_total * case.Hq * case.D * elem  # Q and O
                + layer.seg_table.numel() * 4 + layer.kv_len.numel() * 4 + layer.v2p.numel() * 4)
    tflops = flops / (ms_step * 1e-3) / 1e12
    gbps = io_bytes / (ms_step * 1e-3) / 1e9
    decode = bool((case.q_len * (case.Hq // case.Hkv) <= 16).all())
    kernel = "decode_kernel" if decode else "prefill_kernel"
    if decode:
        achieved = io_bytes / (main_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4)}
    else:
        peak = PEAK_BF16_TFLOPS if case.dtype == "bf16" else PEAK_FP32_TFLOPS
        achieved = flops / (main_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roof["kernel"] = kernel
    roof["kernel_ms"] = round(main_ms, 5)
    roof["traffic"] = load_traffic(case.name, kernel)

    # Cold caches: each step after a 512 MiB read that evicts the L2s and the MALL, so no KV
    # read of one step is served by what the previous step left in cache.
    cold = None
    if args.cold_steps > 0:
        cold_ev = [(HipEvent(), HipEvent()) for _ in range(args.cold_steps)]
        for ev in cold_ev:
            evict()
            layer.attention(q, scale, out=out, events=ev)
        torch.cuda.synchronize()
        cold_ms = float(np.median([a.elapsed_ms(b) for a, b in cold_ev]))
        work = io_bytes / 1e9 if decode else flops / 1e12
        cold_ach = work / (cold_ms * 1e-3)
        cold = {"steps": args.cold_steps, "kernel_ms_median": round(cold_ms, 5),
                "achieved": round(cold_ach, 2), "unit": roof["unit"],
                "frac": round(cold_ach / roof["peak"], 4)}
        assert layer.check() == 0, "device-side error"

    # Dense + mask baseline on the same inputs.
    dense = None
    if importance is not None and not args.no_dense:
        dense = {"skipped": "the dense-plus-mask path has no mask for RETRIEVAL heads"}
    elif not args.no_dense:
        dl = DenseMaskLayer(case.dtype, case.Hq, case.Hkv, case.D, case.ctx_len, case.q_len,
                            case.policy, dev)
        dl.plan()
        dout = torch.empty_like(q)
        for _ in range(args.warmup):
            dl.attention(q, k, v, scale, out=dout)
        torch.cuda.synchronize()
        d0, d1 = HipEvent(), HipEvent()
        d0.record(stream)
        for _ in range(args.steps):
            dl.attention(q, k, v, scale, out=dout)
        d1.record(stream)
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_ms(d1) / args.steps
        dense = {"ms_per_step": round(dense_ms, 5),
                 "speedup": round(dense_ms / ms_step, 3)}

    # CPU oracle on a bounded sample, and parity of the sampled rows.
    threads = len(os.sched_getaffinity(0))
    budget_s = 0.0
    if args.cpu_rows is None:
        # about 15 s of oracle work: rows spread over every (request, query head), up to 64K
        args.cpu_rows, budget_s = 65536, 15.0
    sample, ref_rows, cpu_s, cpu_pairs, cpu_nrows = cpu_oracle_sample(case, args.cpu_rows,
                                                                      importance, budget_s)
    got = out.float().cpu().numpy().astype(np.float64)
    q_row0 = np.concatenate([[0], np.cumsum(case.q_len)[:-1]])
    maxabs, cos_min = 0.0, 1.0
    for (b, hq, toks), ref in zip(sample, ref_rows):
        g = got[q_row0[b] + toks, hq, :]
        maxabs = max(maxabs, float(np.abs(g - ref).max()))
        na, nb = np.linalg.norm(g), np.linalg.norm(ref)
        if na > 0 and nb > 0:
            cos_min = min(cos_min, float((g.ravel() @ ref.ravel()) / (na * nb)))
    cpu_tflops = 4.0 * case.D * cpu_pairs / cpu_s / 1e12

    G = case.Hq // case.Hkv
    dense_tokens = float(np.sum(case.ctx_len)) * case.Hkv
    line = {
        "metric": "visible-KV attention TFLOP/s & HBM GB/s (% roofline) + speedup vs dense+mask",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {"workload": case.name, "B": case.B, "Hq": case.Hq, "Hkv": case.Hkv,
                   "D": case.D, "page_size": case.P, "ctx_len_total": int(case.ctx_len.sum()),
                   "q_len_total": int(case.q_len.sum()),
                   "global_kv_heads": [int(h) for h in np.nonzero(case.policy[:, 0] == 0)[0]],
                   "local_sink_window": [int(case.policy[:, 1].max()),
                                         int(case.policy[:, 2].max())],
                   "local_window_rule": ("context length // %d" % int(case.policy[:, 2].max())
                                         if (case.policy[:, 0] == 2).any() else "fixed"),
                   "gqa_group": G,
                   "page_order": args.page_order,
                   "retrieval_kv_heads": [[int(h), int(case.policy[h, 2])] for h in
                                          np.nonzero(case.policy[:, 0] == 3)[0]]},
        "gbps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "visible_tflop_per_step": round(flops / 1e12, 6),
        "roofline": roof,
        "cold_cache": cold,
        "dense_mask": dense,
        "speedup_vs_dense_mask": dense.get("speedup") if dense else None,
        "build": {"runs": BUILD_RUNS, "seconds": round(build_s, 6),
                  "stream_ms": round(build_ms, 4), "bytes": build_bytes, "gbps_wall": round(build_bytes / build_s / 1e9, 1),
                  "gbps_stream": round(build_bytes / (build_ms * 1e-3) / 1e9, 1)},
        "kv_savings": round(1.0 - rows / dense_tokens, 4),
        "parity_sample": {"rows": cpu_nrows, "max_abs": maxabs, "min_cos": cos_min},
        "cpu_baseline": {"value": float("%.4g" % cpu_tflops), "unit": "TFLOP/s", "cores": threads,
                         "kind": "oracle",
                         "sample": "%d query rows (%d of %d (request, query head) pairs), "
                                   "fp64 numpy (%s BLAS), %.1f s; host has %d CPUs"
                                   % (cpu_nrows, len(sample), case.B * case.Hq, blas_name(),
                                      cpu_s, os.cpu_count() or 0)},
    }
    if args.decode_steps > 0:
        line["decode_append"] = decode_append_leg(args, case, k, v, up, evict, stream, ms_step,
                                                  SegPagedDecoder, HipEvent, decode_tokens,
                                                  free_list, importance)
    if args.build_layers > 0:
        del layer
        line["build_layers"] = build_layers_leg(args.build_layers, case, k, v, evict, stream,
                                                SegPagedLayers, HipEvent, build_ms,
                                                sequential=args.page_order == "sequential")
    print(json.dumps(line), flush=True)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    return 0


def decode_append_leg(args, case, k, v, up, evict, stream, planned_ms, decoder_cls, event_cls,
                      decode_tokens, free_list, importance=None) -> dict:
    """Decode with growth: the workload's context built into a growable layout (pages reserved
    for the steps to come), then warmup + N steps, each appending every request's new token
    and running the table-driven decode on it. Timed with HIP events on the stream: the whole
    loop, and every EVENT_EVERY-th append."""
    import torch
    if int(case.q_len.max()) != 1 or (case.policy[:, 0] == 2).any():
        return {"skipped": "needs a decode workload (one query per request) without "
                           "context-adaptive heads"}
    n_steps, n_warm = args.decode_steps, args.warmup
    total = n_steps + 2 * n_warm
    R = case.B if args.decode_requests <= 0 else min(args.decode_requests, case.B)
    kn, vn, qn = decode_tokens(case, total)
    kn, vn, qn = (up(np.ascontiguousarray(x[:, :R])) for x in (kn, vn, qn))
    ctx, ql = case.ctx_len[:R], case.q_len[:R]
    rows = int(ctx.sum())
    k, v = k[:rows].contiguous(), v[:rows].contiguous()
    reserve = np.full(R, total + n_steps, dtype=np.int32)
    dec = decoder_cls(case.dtype, case.Hq, case.Hkv, case.D, case.P, ctx, ql, reserve,
                      case.policy, k.device)
    dec.build(k, v, free_list(case.seed, dec.n_virt),
              importance=(np.ascontiguousarray(importance[:rows].T)
                          if importance is not None else None))
    dec.plan()
    out = torch.empty_like(qn[0])
    local = case.policy[:, 0] == 1

    def rows_of():
        kl = dec.kv_len.cpu().numpy().astype(np.int64)
        return int(kl[:, local].sum()), int(kl[:, ~local].sum())

    rows0 = rows_of()
    for i in range(n_warm):
        dec.append(kn[i], vn[i])
        dec.decode(qn[i], case.scale, out=out)
    torch.cuda.synchronize()
    rows_w = rows_of()
    ev_a = {i: (event_cls(), event_cls()) for i in range(0, n_steps, EVENT_EVERY)}
    evict()
    e0, e1 = event_cls(), event_cls()
    e0.record(stream)
    for i in range(n_steps):
        j = n_warm + i
        ev = ev_a.get(i)
        if ev:
            ev[0].record(stream)
        dec.append(kn[j], vn[j])
        if ev:
            ev[1].record(stream)
        dec.decode(qn[j], case.scale, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_ms(e1) / n_steps
    append_ms = float(np.mean([a.elapsed_ms(b) for a, b in ev_a.values()]))
    err = dec.check()
    assert err == (0, 0), "device-side error %r" % (err,)
    rows1 = rows_of()
    graph = None
    if args.decode_graph:
        # the same kind of step as replays of one captured graph: the next token's rows and
        # queries are copied into the graph's buffers (on the stream) before each replay
        bufs = [kn[0].clone(), vn[0].clone(), qn[0].clone()]
        g = dec.capture_step(bufs[0], bufs[1], bufs[2], out, case.scale)
        base = n_warm + n_steps
        for i in range(n_warm):
            for buf, src in zip(bufs, (kn, vn, qn)):
                buf.copy_(src[base + i])
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = event_cls(), event_cls()
        g0.record(stream)
        for i in range(n_steps):
            for buf, src in zip(bufs, (kn, vn, qn)):
                buf.copy_(src[(base + n_warm + i) % total])
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        dec.advance(n_warm + n_steps)
        gms = g0.elapsed_ms(g1) / n_steps
        err = dec.check()
        assert err == (0, 0), "device-side error %r" % (err,)
        graph = {"ms_per_step": round(gms, 5), "vs_eager": round(gms / ms, 3)}
    elem = 2 if case.dtype == "bf16" else 4
    # mean stored rows read per step (GLOBAL heads grow by one row a step)
    read_rows = (sum(rows_w) + sum(rows1)) / 2.0
    step_bytes = (2.0 * read_rows * case.D * elem + 2.0 * R * case.Hq * case.D * elem
                  + 2.0 * 2.0 * R * case.Hkv * case.D * elem)  # + the appended rows
    gbps = step_bytes / ((ms - append_ms) * 1e-3) / 1e9
    return {"requests": R, "steps": n_steps, "warmup": n_warm, "ms_per_step": round(ms, 5),
            "append_ms": round(append_ms, 5), "tokens_per_s": round(R / (ms * 1e-3), 1),
            "decode_gbps": round(gbps, 1), "decode_hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
            "vs_planned_step": round(ms / planned_ms, 3) if R == case.B else None,
            "local_rows": [rows0[0], rows1[0]], "other_rows": [rows0[1], rows1[1]],
            "pages_owned": int(dec.n_virt), "graph": graph}


def build_layers_leg(n_layers, case, k, v, evict, stream, layers_cls, event_cls,
                     one_layer_ms, sequential=False) -> dict:
    """Median time of building ``n_layers`` layers of the workload's shape in one call into one
    shared pool: the stacked dense K/V are the workload's layer repeated (values do not change
    the build's work), the policies differ per layer."""
    import torch
    pol = np.stack([np.roll(case.policy, l, axis=0) for l in range(n_layers)])
    layers = layers_cls(case.dtype, n_layers, case.Hq, case.Hkv, case.D, case.P, case.ctx_len,
                        case.q_len, pol, k.device)
    elem = k.element_size()
    need = 2.0 * n_layers * k.numel() * elem + 2.0 * layers.n_virt * case.P * case.D * elem
    free, _ = torch.cuda.mem_get_info()
    if need > 0.8 * free:
        return {"layers": n_layers, "skipped": "needs %.1f GiB of %.1f GiB free"
                % (need / 2 ** 30, free / 2 ** 30)}
    kd = k.unsqueeze(0).expand(n_layers, *k.shape).contiguous()
    vd = v.unsqueeze(0).expand(n_layers, *v.shape).contiguous()
    fl = (np.arange(max(layers.n_virt, 1), dtype=np.int32) if sequential else
          np.random.default_rng(case.seed).permutation(max(layers.n_virt, 1)).astype(np.int32))
    layers.build(kd, vd, fl)
    walls, streams = [], []
    for _ in range(BUILD_RUNS):
        evict()
        torch.cuda.synchronize()
        b0, b1 = event_cls(), event_cls()
        t0 = time.perf_counter()
        b0.record(stream)
        layers.rebuild(kd, vd, fl)
        b1.record(stream)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        streams.append(b0.elapsed_ms(b1))
    wall_s, ms = float(np.median(walls)), float(np.median(streams))
    rows = float(layers.kv_len.sum().item())
    nbytes = 2.0 * 2.0 * rows * case.D * elem  # read + write, K and V
    return {"layers": n_layers, "pages": int(layers.n_virt), "runs": BUILD_RUNS,
            "seconds": round(wall_s, 6), "stream_ms": round(ms, 4), "bytes": nbytes,
            "gbps_wall": round(nbytes / wall_s / 1e9, 1),
            "gbps_stream": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "vs_layers_times_one_layer_build": round(ms / (n_layers * one_layer_ms), 3)}


def blas_name() -> str:
    try:
        return str(np.show_config(mode="dicts")["Build Dependencies"]["blas"]["name"])
    except Exception:  # older numpy: no dict form
        return "unknown"


def gemm_reference() -> int:
    """TFLOP/s of torch.matmul on square bf16 matrices (the vendor GEMM library)."""
    import torch
    out = {}
    for n in (4096, 8192, 16384):
        a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
        b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            a @ b
        torch.cuda.synchronize()
        iters = 20 if n < 16384 else 5
        t0 = time.perf_counter()
        for _ in range(iters):
            a @ b
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / iters
        out[str(n)] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    print(json.dumps({"bf16_gemm_tflops": out, "peak": PEAK_BF16_TFLOPS}), flush=True)
    return 0


def _main_kernel_counters(d: str, kernel: str) -> dict:
    """Mean of every counter over the paged-mode dispatches of `kernel` in one --pmc run."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under " + d)
    vals = {}
    for r in csv.DictReader(open(files[0])):
        n = r["Kernel_Name"]
        if kernel + "<" in n and (kernel == "build_kernel" or ", 0>" in n):
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("%s: no %s dispatch in %s" % (kernel, kernel, d))
    return {k: float(np.mean(v)) for k, v in vals.items()}


def write_counters(args) -> int:
    """Per-dispatch counter means of the workload's main kernel, plus what they imply: the
    matrix-core busy share (MfmaUtil), bf16 MFMA FLOPs per dispatch against the FLOPs of the
    visible (query, key) pairs, and instruction counts per wave and 64-key KV step."""
    from workloads import config_case
    case = config_case(args.config, with_tensors=False)
    decode = bool((case.q_len * (case.Hq // case.Hkv) <= 16).all())
    kernel = "decode_kernel" if decode else "prefill_kernel"
    if args.counters_kernel == "build":
        kernel = "build_kernel"
    counters = {}
    for d in args.counters_from:
        counters.update(_main_kernel_counters(d, kernel))
    rec = {"kernel": kernel, "counters": {k: round(v, 3) for k, v in sorted(counters.items())}}
    flops = 4.0 * case.D * visible_counts(case).sum() * (case.Hq // case.Hkv)
    if kernel != "build_kernel":
        rec["visible_flops_per_launch"] = flops
    if "MfmaFlopsBF16" in counters and kernel != "build_kernel":
        rec["mfma_bf16_flops_per_launch"] = counters["MfmaFlopsBF16"]
        rec["mfma_flops_over_visible"] = round(counters["MfmaFlopsBF16"] / flops, 4)
    if "MfmaUtil" in counters:
        rec["mfma_busy_pct"] = round(counters["MfmaUtil"], 2)
    if "SQ_WAVES" in counters and "SQ_INSTS_MFMA" in counters and kernel == "prefill_kernel":
        # every prefill wave issues 32 bf16 MFMAs (32x32x16) per 64-key step
        steps = counters["SQ_INSTS_MFMA"] / 32.0
        rec["per_wave_step"] = {k[len("SQ_INSTS_"):].lower(): round(counters[k] / steps, 1)
                                for k in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
                                          "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32")
                                if k in counters}
    if "GRBM_GUI_ACTIVE" in counters:
        # GRBM_GUI_ACTIVE adds up the 8 XCDs' clocks; the _avr counters average over the
        # block's instances, the _sum counters add them up (TD: one per CU, 256 CUs)
        cyc = counters["GRBM_GUI_ACTIVE"] / 8.0
        mp = {}
        if "TA_BUSY_avr" in counters:
            mp["ta_busy_pct"] = round(100.0 * counters["TA_BUSY_avr"] / cyc, 1)
        if "TD_TD_BUSY_sum" in counters:
            mp["td_busy_pct"] = round(100.0 * counters["TD_TD_BUSY_sum"] / 256.0 / cyc, 1)
        if "TCC_BUSY_avr" in counters:
            mp["l2_busy_pct"] = round(100.0 * counters["TCC_BUSY_avr"] / cyc, 1)
        if "TCC_HIT_sum" in counters and "TCC_MISS_sum" in counters:
            mp["l2_hit_pct"] = round(100.0 * counters["TCC_HIT_sum"] /
                                     (counters["TCC_HIT_sum"] + counters["TCC_MISS_sum"]), 1)
        if "TA_ADDR_STALLED_BY_TC_CYCLES_sum" in counters:
            mp["ta_addr_stalled_by_l1_pct"] = round(
                100.0 * counters["TA_ADDR_STALLED_BY_TC_CYCLES_sum"] / 256.0 / cyc, 1)
        if "TCP_TCR_TCP_STALL_CYCLES_sum" in counters:
            mp["l1_stalled_by_l2_pct"] = round(
                100.0 * counters["TCP_TCR_TCP_STALL_CYCLES_sum"] / 256.0 / cyc, 1)
        rec["memory_path"] = mp
    rec["source_hash"] = source_hash()
    path = os.path.join(ROOT, "profiles", "counters.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data.setdefault(case.name, {})[kernel] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({case.name: rec}))
    return 0


COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _counter_rows(d: str, counter: str):
    """(kernel name, value) per dispatch of one rocprofv3 --pmc csv run directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under " + d)
    out = []
    for r in csv.DictReader(open(files[0])):
        if r["Counter_Name"] == counter:
            out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def write_traffic(args) -> int:
    """HBM bytes per launch of the workload's main kernel from FETCH_SIZE / WRITE_SIZE runs.

    Both counters are in KiB per dispatch. Each is scaled by the factor that makes it read
    right for the largest device-to-device copy in the same run (copy_bytes read and written).
    """
    from workloads import config_case
    case = config_case(args.config, with_tensors=False)
    decode = bool((case.q_len * (case.Hq // case.Hkv) <= 16).all())
    kernel = "decode_kernel" if decode else "prefill_kernel"
    copy_bytes = float(args.copy_calibration << 20)
    if copy_bytes <= 0:
        raise SystemExit("--traffic-from needs --copy-calibration MIB of the counter runs")
    rec = {"kernel": kernel, "copy_bytes": copy_bytes}
    for d, counter in zip(args.traffic_from, ("FETCH_SIZE", "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        main = [v for n, v in rows if kernel + "<" in n and ", 0>" in n]
        copy = [v for n, v in rows if COPY_KERNEL in n]
        if not main or not copy:
            raise SystemExit("%s: main or copy kernel missing in %s" % (counter, d))
        per = float(np.mean(main))
        cal = max(copy)
        factor = copy_bytes / (cal * 1024.0)
        key = "fetch" if counter == "FETCH_SIZE" else "write"
        rec[key + "_kib_per_launch"] = round(per, 1)
        rec[key + "_copy_kib"] = round(cal, 1)
        rec[key + "_factor"] = round(factor, 4)
        rec[key + "_bytes"] = per * 1024.0 * factor
    rec["bytes_per_launch"] = round(rec.pop("fetch_bytes") + rec.pop("write_bytes"))
    rec["source_hash"] = source_hash()
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data.setdefault(case.name, {})[kernel] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({case.name: rec}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
