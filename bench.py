#!/usr/bin/env python3
"""CSA2 decode benchmark on one MI355X.

Workload (the 128K decode configuration): a Full -> Reindex -> Reuse layer group over one
shared cache, 16 sequences x 131072 cached entries.  Indexer: 32 heads x 64 dims, E4M3
keys with a per-token fp32 scale, bf16 queries, head weights U(0,1); Top-512; main KV
512-dim FP4 E2M1 with per-channel fp32 scales (values N(0,1) plus 1 % of channels x 8);
64 attention heads, bf16 query and output.  Every layer draws its own queries/weights.

A step is one pass of the whole decode path of the group (indexer scores, Top-K, gather +
FP4 dequant + attention, for all three layers).  Two protocols are timed:

* flushed (the headline): every layer is its own C-ABI call, a 512 MiB buffer is written
  before each layer (evicting the 256 MB Infinity Cache and the L2s, as the other layers of
  a real model would), and the step time is the sum of the per-layer HIP-event times.
* warm: the whole group as one csa2_layer_group call, cache copies rotated between steps.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import compressed_sparse_attention_csa2_amd as csa2  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 512 << 20  # written before every flushed layer: twice the 256 MB Infinity Cache
SCORE_SOURCES = ("compressed_sparse_attention_csa2_amd/csrc/score.hip", "compressed_sparse_attention_csa2_amd/csrc/common.hpp",
                 "compressed_sparse_attention_csa2_amd/csrc/launch.hpp",
                 "compressed_sparse_attention_csa2_amd/csrc/score_dev.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_fp8_group128k_hbm_traffic.md")
METRIC = "CSA2 decode queries/s + achieved HBM GB/s (% of peak) at 128K context"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Flusher:
    """Writes a 512 MiB device buffer (a plain fill): afterwards neither the Infinity Cache
    nor any L2 holds the data of the layer before."""

    def __init__(self):
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(1 + self.n % 200)


def host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return dict(cpu_model=model, nproc=os.cpu_count(), affinity_cpus=affinity)


def layer_calls(wl, c, layers, out_dtype=torch.bfloat16):
    """One C-ABI call per layer of the group, for the flushed protocol: a Full or Reindex
    layer is a one-layer csa2_layer_group (without a candidate pool a Reindex layer takes
    exactly the steps of a Full layer over the shared cache: every entry scored with its own
    query, a fresh Top-K, attention); a Reuse layer is csa2_sparse_attend on the indices of
    the most recent indexing layer, unchanged."""
    calls, last_idx = [], None
    for L in layers:
        if L["mode"] != "reuse":
            d = dict(mode="full", q_idx=L["q_idx"], w=L["w"], q_attn=L["q_attn"])
            plan = csa2.GroupPlan([d], csa2.GroupCache(c["n_keys"], c["codes"], c["scales"], c["k8"], c["ks"], wl.K,
                                                       wl.softmax_scale), out_dtype=out_dtype)
            calls.append(plan.run)
            last_idx = d["idx"]
        else:
            out = torch.empty((wl.B, 1, wl.Hq, wl.D), dtype=out_dtype, device="cuda")
            lse = torch.empty((wl.B, 1, wl.Hq), dtype=torch.float32, device="cuda")

            def reuse(q=L["q_attn"], idx=last_idx, out=out, lse=lse):
                csa2.sparse_attend(q, c["codes"], c["scales"], idx, wl.softmax_scale, out=out, lse=lse)
            calls.append(reuse)
    return calls


def time_flushed(calls, steps, warmup, flush):
    """Flushed protocol: before every layer the flush buffer is written; each layer's call
    is bracketed by HIP events on the launching stream (torch's current stream, which the
    library launches on).  Returns (mean step ms = mean over steps of the summed layer
    times, per-layer mean ms, wall seconds of the whole timed loop incl. the flushes)."""
    n = len(calls)
    for _ in range(warmup):
        for f in calls:
            flush()
            f()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
           for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        for i, f in enumerate(calls):
            flush()
            evs[s][i][0].record()
            f()
            evs[s][i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[a.elapsed_time(b) for a, b in row] for row in evs])  # [steps][layers] ms
    return float(per.sum(axis=1).mean()), [float(x) for x in per.mean(axis=0)], wall


def time_flushed_by_difference(calls, steps, flush):
    """The flushed layers timed by difference (as time_cold): per layer, HIP events around
    (flush, layer call) and around a flush alone, interleaved; the mean difference is the
    layer's GPU time without the event pair's own dispatch.  Returns (step ms, per-layer ms)."""
    n = len(calls)
    both, alone = np.zeros((steps, n)), np.zeros((steps, n))
    for s in range(steps):
        for i, f in enumerate(calls):
            for sink, run in ((both, f), (alone, None)):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                flush()
                if run is not None:
                    run()
                b.record()
                torch.cuda.synchronize()
                sink[s, i] = a.elapsed_time(b)
    per = both.mean(axis=0) - alone.mean(axis=0)
    return float(per.sum()), [float(x) for x in per]


def time_warm(plans, steps, warmup):
    for s in range(warmup):
        plans[s % len(plans)].run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        plans[s % len(plans)].run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def stream_ceiling(buf, flush, reps=12):
    """Read rate (GB/s) of the library's streaming probe over `buf` from HBM (a flush before
    every read), best over a few grid sizes: the practical ceiling for a kernel that reads
    these bytes once."""
    best = 0.0
    sink = torch.empty(1, dtype=torch.int32, device="cuda")
    nbytes = buf.numel() * buf.element_size()
    for blocks in (256, 512, 1024, 2048):
        # timed like the score kernel it is compared with (by difference, see time_cold)
        ms, _, _ = time_cold(lambda: csa2.stream_probe(buf, blocks, sink), flush, reps)
        best = max(best, nbytes / (ms / 1e3) / 1e9)
    return best


def time_cold(launch, flush, reps):
    """A launch on a cold cache, timed with HIP events on the launching stream two ways:
    directly (events around the launch, after a flush), and by difference (events around
    flush + launch, and around a flush alone, interleaved): the difference cancels the event
    pair's own dispatch, about 3 us on this GPU, and matches the kernel trace's duration.
    Returns (difference mean ms, direct mean ms, direct median ms)."""
    direct, both, alone = [], [], []
    for _ in range(reps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize()
        direct.append(a.elapsed_time(b))
        for sink, with_launch in ((both, True), (alone, False)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            flush()
            if with_launch:
                launch()
            b.record()
            torch.cuda.synchronize()
            sink.append(a.elapsed_time(b))
    return float(np.mean(both) - np.mean(alone)), float(np.mean(direct)), float(np.median(direct))


def score_roofline(wl, c, L, reps, flush):
    """The decode score kernel (one launch per csa2_index_score call) on a cold cache: a
    flush before every launch, each launch bracketed by HIP events on the launching stream.
    Algorithmic bytes per launch: every key's 64 code bytes and 4-byte scale read once, plus
    the query and head weights (the kernel also writes one fp32 score per key, which is
    traffic beyond the algorithm and shows in the counted traffic instead)."""
    out = torch.empty((wl.B, 1, wl.N), dtype=torch.float32, device="cuda")

    def launch():
        csa2.index_score(csa2.PREC_FP8, L["q_idx"], L["w"], c["k8"], c["ks"], c["n_keys"], scores=out)

    for _ in range(3):
        flush()
        launch()
    torch.cuda.synchronize()
    mean_ms, direct_ms, direct_median = time_cold(launch, flush, reps)
    # the same kernel back to back without a flush (its keys partly in the Infinity Cache)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        launch()
    b.record()
    torch.cuda.synchronize()
    warm_ms = a.elapsed_time(b) / reps
    nbytes = wl.B * wl.N * (wl.dk + 4) + wl.B * wl.H * (wl.dk * 2 + 4)
    return dict(bytes_per_launch=nbytes, kernel_ms_mean=mean_ms, kernel_ms_direct=direct_ms,
                kernel_ms_direct_median=direct_median, warm_kernel_ms_mean=float(warm_ms),
                achieved=nbytes / (mean_ms / 1e3) / 1e9)


def build_device_cache(wl, copies, kv_fmt=csa2.FMT_FP4_PER_CHANNEL, key_fmt=csa2.FMT_FP8_PER_TOKEN):
    """Quantise the workload's cache on the GPU (one sequence at a time) and clone it.  The
    main KV takes one fp32 scale per channel, or (FMT_FP4_G16) one E4M3 scale per 16
    channels of each entry; the indexer keys are E4M3, or (FMT_FP4_PER_TOKEN) E2M1, with
    one scale per row."""
    B, N, D, dk = wl.B, wl.N, wl.D, wl.dk
    codes = torch.empty((B, N, D // 2), dtype=torch.uint8, device="cuda")
    if kv_fmt == csa2.FMT_FP4_G16:
        scales = torch.empty((B, N, D // 16), dtype=torch.uint8, device="cuda")
    else:
        scales = torch.empty((B, D), dtype=torch.float32, device="cuda")
    k8 = torch.empty((B, N, dk if key_fmt == csa2.FMT_FP8_PER_TOKEN else dk // 2), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, N), dtype=torch.float32, device="cuda")
    for b in range(B):
        x = torch.from_numpy(wl.main_kv(b)).to("cuda")
        csa2.quantize_kv(kv_fmt, x[None], codes[b:b + 1], scales[b:b + 1])
        kf = torch.from_numpy(wl.index_keys(b)).to("cuda")
        csa2.quantize_kv(key_fmt, kf[None], k8[b:b + 1], ks[b:b + 1])
        torch.cuda.synchronize()
        del x, kf
    n_keys = torch.full((B,), N, dtype=torch.int32, device="cuda")
    caches = [dict(codes=codes, scales=scales, k8=k8, ks=ks, n_keys=n_keys)]
    for _ in range(copies - 1):
        caches.append({k: v.clone() for k, v in caches[0].items()})
    return caches


def layer_inputs(wl):
    layers = []
    for i, m in enumerate(wl.modes):
        layers.append(dict(mode=m,
                           q_idx=torch.from_numpy(wl.index_query(i)).to(torch.bfloat16).cuda(),
                           w=torch.from_numpy(wl.head_weights(i)).cuda(),
                           q_attn=torch.from_numpy(wl.attn_query(i)).to(torch.bfloat16).cuda()))
    return layers


def algorithmic_bytes(wl):
    """Bytes the group must move at least once: per indexing layer the key
    scan (64 B key + 4 B scale per entry) and per layer the gathered FP4 rows, their
    scales, the query, the output and the indices."""
    B, N, K, D, Hq = wl.B, wl.N, wl.K, wl.D, wl.Hq
    n_index = sum(1 for m in wl.modes if m != "reuse")
    scan = B * N * (wl.dk + 4)
    q_idx = B * wl.H * wl.dk * 2 + B * wl.H * 4
    per_layer_attend = B * K * (D // 2) + B * D * 4 + B * Hq * D * 2 * 2 + B * K * 4 + B * Hq * 4
    return n_index * (scan + q_idx + B * K * 4) + len(wl.modes) * per_layer_attend


def score_sources_sha256():
    """Digest of the sources the score kernel is built from (the HBM-traffic figures below
    hold only for the kernel they were counted on)."""
    import hashlib
    h = hashlib.sha256()
    for rel in SCORE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counted_traffic():
    """HBM bytes per score launch from the committed rocprofv3 --pmc summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by the same counter's reading on a copy of known size), or
    None when the summary is absent or the kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_sources_sha256") != score_sources_sha256():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(nbytes, reps=5):
    """A plain device copy of known size (read nbytes, write nbytes): the calibration
    kernel for the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def cpu_baseline(wl, seqs):
    """The CPU oracle, as it stands, on the same workload restricted to `seqs` sequences
    (the cache build is setup; the timed part is the group's decode path)."""
    import oracle
    sub = workloads.workload(wl.name, B=seqs)
    ks, k8s, codes, scales = [], [], [], []
    for b in range(seqs):
        c, s = oracle.quantize_fp4(sub.main_kv(b)[None])
        codes.append(c[0]); scales.append(s[0])
        k8, kss = oracle.quantize_fp8(sub.index_keys(b)[None])
        k8s.append(k8[0]); ks.append(kss[0])
    cache = dict(k=np.stack(k8s), k_scale=np.stack(ks), n_keys=np.full(seqs, sub.N, np.int32),
                 codes=np.stack(codes), scales=np.stack(scales))
    layers = [dict(mode=m, q_idx=sub.index_query(i), w=sub.head_weights(i), q_attn=sub.attn_query(i))
              for i, m in enumerate(sub.modes)]
    t0 = time.perf_counter()
    oracle.layer_group(layers, cache, oracle.PREC_FP8, sub.K, sub.softmax_scale)
    dt = time.perf_counter() - t0
    res = dict(value=seqs / dt, unit="queries/s", cores=oracle.num_threads(), kind="oracle",
               sample="%d of %d sequences of the same workload (N=%d, all %d layers); %.2f s" %
                      (seqs, wl.B, wl.N, len(wl.modes), dt))
    res.update(host_info())
    return res


def run_prefill(args):
    """Chunked prefill (262144 cached entries + 4096 new tokens, one sequence): a step is
    the whole path for the new tokens - FP4 (GIVEN scales) and E4M3 append of their main KV
    and indexer keys, causal fp8 scoring of every new token against all visible entries,
    Top-512 per token, sparse attention of 64 bf16 heads per token."""
    wl = workloads.WORKLOADS["prefill"]
    Nc, T, D, dk = wl.N, wl.T, wl.D, wl.dk
    n_max = Nc + T
    log("building the cached part (%d entries) ..." % Nc)
    codes = torch.zeros((1, n_max, D // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((1, D), dtype=torch.float32, device="cuda")
    k8 = torch.zeros((1, n_max, dk), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((1, n_max), dtype=torch.float32, device="cuda")
    csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, torch.from_numpy(wl.main_kv(0)[None]).cuda(), codes, scales)
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, torch.from_numpy(wl.index_keys(0)[None]).cuda(), k8, ks)
    new = torch.from_numpy(wl.new_kv()).to(torch.bfloat16).cuda()
    newk = torch.from_numpy(wl.new_index_keys()).cuda()
    n0 = torch.tensor([Nc], dtype=torch.int32, device="cuda")
    n_keys = torch.tensor([n_max], dtype=torch.int32, device="cuda")
    q_limit = (Nc + torch.arange(T, dtype=torch.int32, device="cuda"))[None].contiguous()
    q = torch.from_numpy(wl.index_query()).to(torch.bfloat16).cuda()
    w = torch.from_numpy(wl.head_weights()).cuda()
    qa = torch.from_numpy(wl.attn_query()).to(torch.bfloat16).cuda()
    idx = torch.empty((1, T, wl.K), dtype=torch.int32, device="cuda")
    out = torch.empty((1, T, wl.Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, T, wl.Hq), dtype=torch.float32, device="cuda")

    def step():
        csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, new, codes, scales, scale_policy=csa2.SCALE_GIVEN, n0=n0)
        csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, newk, k8, ks, n0=n0)
        csa2.index_topk(csa2.PREC_FP8, q, w, k8, ks, n_keys, wl.K, q_limit=q_limit, idx=idx)
        csa2.sparse_attend(qa, codes, scales, idx, wl.softmax_scale, out=out, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    # the indexer's Top-K as the step runs it: events around back-to-back csa2_index_topk
    # calls (the query quantisation, the many-row scan that lists each region's candidates,
    # and the selection), so the fp8 MFMA rate below counts the selection's time as well
    reps = 5
    csa2.index_topk(csa2.PREC_FP8, q, w, k8, ks, n_keys, wl.K, q_limit=q_limit, idx=idx)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        csa2.index_topk(csa2.PREC_FP8, q, w, k8, ks, n_keys, wl.K, q_limit=q_limit, idx=idx)
    e1.record()
    torch.cuda.synchronize()
    score_ms = e0.elapsed_time(e1) / reps
    pairs = sum(Nc + t + 1 for t in range(T))
    flops = 2 * wl.H * dk * pairs
    tflops = flops / (score_ms / 1e3) / 1e12
    res = {
        "metric": "CSA2 chunked-prefill new tokens/s", "value": round(T / (ms_step / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": "prefill: 262144 cached + 4096 new tokens, causal, indexer 32x64 E4M3, Top-512, "
                               "FP4 E2M1 main KV D=512, 64 heads bf16", "global_batch": 1, "seq_len": n_max},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": 5000.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 5000.0, 4), "traffic": None,
                     "kernel": "k_quant_query + k_score_fp8_rows_list + k_topk_select (one csa2_index_topk call)",
                     "kernel_ms_mean": round(score_ms, 4), "flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline_prefill(wl, args.cpu_rows)
    print(json.dumps(res), flush=True)


def cpu_baseline_prefill(wl, rows):
    """The CPU oracle on a bounded sample of the chunked-prefill step: the append of all
    4096 new tokens (FP4 with the cache's scales, E4M3 keys), then for `rows` new tokens
    spread over the chunk the causal score against every visible entry, Top-512 and the
    attention; reported as new tokens per second of those rows."""
    import oracle
    Nc, T = wl.N, wl.T
    n_max = Nc + T
    pick = np.linspace(0, T - 1, rows).astype(np.int64)
    cr, sr = oracle.quantize_fp4(wl.main_kv(0)[None], n_max=n_max)
    kr, ksr = oracle.quantize_fp8(wl.index_keys(0)[None], n_max=n_max)
    t0 = time.perf_counter()
    oracle.quantize_fp4(wl.new_kv(), n_max=n_max, n0=np.array([Nc], np.int32), scales=sr, codes=cr)
    oracle.quantize_fp8(wl.new_index_keys(), n_max=n_max, n0=np.array([Nc], np.int32), codes=kr, scales=ksr)
    t_append = time.perf_counter() - t0
    q, w, qa = wl.index_query()[:, pick], wl.head_weights()[:, pick], wl.attn_query()[:, pick]
    ql = (Nc + pick).astype(np.int32)[None]
    t1 = time.perf_counter()
    s = oracle.index_score(oracle.PREC_FP8, q, w, kr, ksr, np.array([n_max], np.int32), q_limit=ql)
    idx = oracle.topk(s, wl.K)
    oracle.sparse_attend(qa, cr, sr, idx, wl.softmax_scale)
    t_rows = time.perf_counter() - t1
    dt = t_rows + t_append * rows / T
    res = dict(value=rows / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
               sample="%d of the %d new tokens (rows spread over the chunk: causal score against every visible "
                      "entry, Top-%d, attention; %.2f s) plus the append of the whole chunk (%.2f s) counted "
                      "pro rata" % (rows, T, wl.K, t_rows, t_append))
    res.update(host_info())
    return res


def run_full64k(args):
    """The single-layer 64K decode configuration: a Full layer over 16 sequences x 65536
    entries (score, Top-512, FP4 gather + attention).  Flushed protocol as the headline (the
    512 MiB flush before every step); the warm number (3 rotated cache copies) beside it."""
    wl = workloads.WORKLOADS["full64k"]
    log("building cache (%d copies) ..." % args.copies)
    caches = build_device_cache(wl, args.copies)
    layers = layer_inputs(wl)
    flush = Flusher()
    ms_step, per_layer, wall = time_flushed(layer_calls(wl, caches[0], layers), args.steps, args.warmup, flush)
    plans = [csa2.GroupPlan([dict(L) for L in layers],
                            csa2.GroupCache(c["n_keys"], c["codes"], c["scales"], c["k8"], c["ks"], wl.K,
                                            wl.softmax_scale), out_dtype=torch.bfloat16) for c in caches]
    warm_ms = time_warm(plans, args.steps, args.warmup)
    alg = algorithmic_bytes(wl)
    gbs = alg / (ms_step / 1e3) / 1e9
    rf = score_roofline(wl, caches[0], layers[0], args.score_reps, flush)
    ceil = stream_ceiling(caches[0]["k8"], flush)
    res = {
        "metric": "CSA2 decode queries/s at 64K context (single Full layer)", "value": round(wl.B / (ms_step / 1e3), 1),
        "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": "full64k: Full decode, B=16, N=65536, indexer 32x64 E4M3, Top-512, FP4 E2M1 main KV "
                               "D=512, 64 heads bf16", "global_batch": wl.B, "seq_len": wl.N,
                   "protocol": "flushed: 512 MiB written before the layer, HIP-event time of the call"},
        "step_algorithmic_bytes": alg, "step_achieved_GBps": round(gbs, 1),
        "step_pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "step_pct_stream_ceiling": round(100 * gbs / ceil, 2),
        "warm_ms_per_step": round(warm_ms, 5), "stream_ceiling_GBps": round(ceil, 1),
        "roofline": {"bound": "hbm", "achieved": round(rf["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(rf["achieved"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "frac_of_stream_ceiling": round(rf["achieved"] / ceil, 4),
                     "kernel": "k_score_fp8 (cold: flushed before each launch)",
                     "kernel_ms_mean": round(rf["kernel_ms_mean"], 5),
                     "kernel_ms_direct": round(rf["kernel_ms_direct"], 5), "bytes_per_launch": rf["bytes_per_launch"]}}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seqs)
    print(json.dumps(res), flush=True)


DECODER_MODES = ["full"] + ["reuse"] * 3 + (["reindex"] + ["reuse"] * 3) * 4
DECODER_POOL = (8, 2048)


def run_decoder128k(args):
    """The decoder's layer schedule (Full, 3 Reuse, then 4 x [Reindex, 3 Reuse]; 20 layers)
    at 128K context, 16 sequences: the Full layer scans all 131072 entries and also keeps its
    best 2048 blocks of 8 entries (by block maximum) as the candidate pool; every Reindex
    layer scores only the pool's 16384 positions.  The same schedule without the pool (every
    Reindex layer scans everything) is timed beside it."""
    wl = workloads.WORKLOADS["group128k"]
    log("building cache (%d copies) ..." % args.copies)
    caches = build_device_cache(wl, args.copies)
    layers = []
    for i, m in enumerate(DECODER_MODES):
        layers.append(dict(mode=m, q_idx=torch.from_numpy(wl.index_query(i)).to(torch.bfloat16).cuda(),
                           w=torch.from_numpy(wl.head_weights(i)).cuda(),
                           q_attn=torch.from_numpy(wl.attn_query(i)).to(torch.bfloat16).cuda()))

    def timed(pool):
        plans = [csa2.GroupPlan([dict(L) for L in layers],
                                csa2.GroupCache(c["n_keys"], c["codes"], c["scales"], c["k8"], c["ks"], wl.K,
                                                wl.softmax_scale, pool=pool), out_dtype=torch.bfloat16)
                 for c in caches]
        for s in range(args.warmup):
            plans[s % len(plans)].run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            plans[s % len(plans)].run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    ms_step = timed(DECODER_POOL)
    flat_ms = timed(None)
    B, N, K, D, Hq = wl.B, wl.N, wl.K, wl.D, wl.Hq
    C = DECODER_POOL[0] * DECODER_POOL[1]
    n_reindex = DECODER_MODES.count("reindex")
    q_idx = B * wl.H * wl.dk * 2 + B * wl.H * 4
    attend = B * K * (D // 2) + B * D * 4 + B * Hq * D * 2 * 2 + B * K * 4 + B * Hq * 4
    # Full: the scan, its scores' block maxima (read back once) and the pool written; Reindex:
    # the pool read and its entries' keys and scales
    alg = (B * N * (wl.dk + 4) + B * N * 4 + B * C * 4 + q_idx + B * K * 4) + \
        n_reindex * (B * C * (4 + wl.dk + 4) + q_idx + B * K * 4) + len(DECODER_MODES) * attend
    gbs = alg / (ms_step / 1e3) / 1e9
    print(json.dumps({
        "metric": "CSA2 decode queries/s at 128K context (decoder schedule with the candidate pool)",
        "value": round(B / (ms_step / 1e3), 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": "decoder128k: Full, 3 Reuse, 4 x [Reindex, 3 Reuse] (20 layers), B=16, N=131072, "
                               "pool of 2048 blocks x 8, indexer 32x64 E4M3, Top-512, FP4 E2M1 main KV D=512, "
                               "64 heads bf16", "global_batch": B, "seq_len": N, "layers": DECODER_MODES,
                   "pool": list(DECODER_POOL), "cache_copies": args.copies},
        "step_algorithmic_bytes": alg, "step_achieved_GBps": round(gbs, 1),
        "step_pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "no_pool_ms_per_step": round(flat_ms, 5)}), flush=True)


def run_group128k_g16(args):
    """The 128K decode group (Full -> Reindex -> Reuse, 16 x 131072, Top-512) with the
    pages' FP4 layout: one E4M3 scale per 16 channels of each entry (288 B per entry
    instead of 256 B plus a per-sequence scale row)."""
    wl = workloads.WORKLOADS["group128k"]
    log("building cache (%d copies) ..." % args.copies)
    caches = build_device_cache(wl, args.copies, csa2.FMT_FP4_G16)
    layers = layer_inputs(wl)
    plans = [csa2.GroupPlan([dict(L) for L in layers],
                            csa2.GroupCache(c["n_keys"], c["codes"], c["scales"], c["k8"], c["ks"], wl.K,
                                            wl.softmax_scale), out_dtype=torch.bfloat16) for c in caches]
    for s in range(args.warmup):
        plans[s % len(plans)].run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        plans[s % len(plans)].run()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    # as algorithmic_bytes, with 32 B of group scales gathered per entry instead of the
    # per-sequence scale row
    B, K, D = wl.B, wl.K, wl.D
    alg = algorithmic_bytes(wl) + len(wl.modes) * (B * K * (D // 16) - B * D * 4)
    gbs = alg / (ms_step / 1e3) / 1e9
    print(json.dumps({
        "metric": "CSA2 decode queries/s at 128K context (FP4 with one E4M3 scale per 16 channels)",
        "value": round(B / (ms_step / 1e3), 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": "group128k_g16: Full->Reindex->Reuse decode, B=16, N=131072, indexer 32x64 E4M3, "
                               "Top-512, FP4 E2M1 main KV D=512 with one E4M3 scale per 16 channels (288 B/entry), "
                               "64 heads bf16", "global_batch": B, "seq_len": wl.N, "layers": list(wl.modes),
                   "cache_copies": args.copies},
        "step_algorithmic_bytes": alg, "step_achieved_GBps": round(gbs, 1),
        "step_pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}), flush=True)


def run_group128k_swa(args):
    """The 128K decode group (Full -> Reindex -> Reuse, 16 x 131072, Top-512) where every
    layer also attends to its own sliding window of the last 128 tokens (E4M3 rows with one
    fp32 scale each) in the same softmax as its selected entries."""
    wl = workloads.WORKLOADS["group128k"]
    W = 128
    log("building cache (%d copies) ..." % args.copies)
    caches = build_device_cache(wl, args.copies)
    layers = layer_inputs(wl)
    gen = torch.Generator(device="cuda").manual_seed(7)
    end = torch.full((wl.B, 1), W, dtype=torch.int32, device="cuda")
    for i, L in enumerate(layers):   # every layer its own window cache
        x = torch.randn((wl.B, W, wl.D), generator=gen, device="cuda")
        wc = torch.empty((wl.B, W, wl.D), dtype=torch.uint8, device="cuda")
        ws = torch.empty((wl.B, W), dtype=torch.float32, device="cuda")
        csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, x, wc, ws)
        L["swa"] = csa2.Swa(wc, ws, end, W)
    plans = [csa2.GroupPlan([dict(L) for L in layers],
                            csa2.GroupCache(c["n_keys"], c["codes"], c["scales"], c["k8"], c["ks"], wl.K,
                                            wl.softmax_scale), out_dtype=torch.bfloat16) for c in caches]
    for s in range(args.warmup):
        plans[s % len(plans)].run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        plans[s % len(plans)].run()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    B, D = wl.B, wl.D
    alg = algorithmic_bytes(wl) + len(wl.modes) * B * W * (D + 4)
    gbs = alg / (ms_step / 1e3) / 1e9
    print(json.dumps({
        "metric": "CSA2 decode queries/s at 128K context (Top-512 plus a 128-token sliding window per layer)",
        "value": round(B / (ms_step / 1e3), 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": "group128k_swa: Full->Reindex->Reuse decode, B=16, N=131072, indexer 32x64 E4M3, "
                               "Top-512 + a 128-entry E4M3 sliding window per layer in one softmax, FP4 E2M1 main "
                               "KV D=512, 64 heads bf16", "global_batch": B, "seq_len": wl.N,
                   "layers": list(wl.modes), "window": W, "cache_copies": args.copies},
        "step_algorithmic_bytes": alg, "step_achieved_GBps": round(gbs, 1),
        "step_pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}), flush=True)


def run_group128k_fp4idx(args):
    """The 128K decode group (Full -> Reindex -> Reuse, 16 x 131072, Top-512) with the 4-bit
    indexer: E2M1 keys with one fp32 scale per row (36 B per key instead of 68) and the
    query quantised to E2M1 per head, scored on the FP4 form of the MFMA."""
    wl = workloads.WORKLOADS["group128k"]
    log("building cache (%d copies) ..." % args.copies)
    caches = build_device_cache(wl, args.copies, key_fmt=csa2.FMT_FP4_PER_TOKEN)
    layers = layer_inputs(wl)
    plans = [csa2.GroupPlan([dict(L) for L in layers],
                            csa2.GroupCache(c["n_keys"], c["codes"], c["scales"], c["k8"], c["ks"], wl.K,
                                            wl.softmax_scale, prec=csa2.PREC_FP4), out_dtype=torch.bfloat16)
             for c in caches]
    for s in range(args.warmup):
        plans[s % len(plans)].run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        plans[s % len(plans)].run()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    B, N = wl.B, wl.N
    n_index = sum(1 for m in wl.modes if m != "reuse")
    alg = algorithmic_bytes(wl) - n_index * B * N * (wl.dk // 2)    # 32 of the 64 key bytes
    gbs = alg / (ms_step / 1e3) / 1e9
    print(json.dumps({
        "metric": "CSA2 decode queries/s at 128K context (4-bit indexer)", "value": round(B / (ms_step / 1e3), 1),
        "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4+bf16", "data": "synthetic",
        "config": {"workload": "group128k_fp4idx: Full->Reindex->Reuse decode, B=16, N=131072, indexer 32x64 E2M1 "
                               "(per-row scale), Top-512, FP4 E2M1 main KV D=512, 64 heads bf16",
                   "global_batch": B, "seq_len": N, "layers": list(wl.modes), "cache_copies": args.copies},
        "step_algorithmic_bytes": alg, "step_achieved_GBps": round(gbs, 1),
        "step_pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}), flush=True)


def run_hier1m(args):
    """The 1M-entry two-level configuration (one sequence): coarse keys (64-entry block
    means, built once, not timed) -> score 16384 coarse keys -> top-256 blocks -> exact
    scores of their 16384 entries -> Top-1024 -> attention over the 1024 entries."""
    wl = workloads.WORKLOADS["hier1m"]
    n = wl.N
    k8 = torch.empty((1, n, wl.dk), dtype=torch.uint8, device="cuda")
    ks = torch.empty((1, n), dtype=torch.float32, device="cuda")
    codes = torch.empty((1, n, wl.D // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((1, wl.D), dtype=torch.float32, device="cuda")
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, torch.from_numpy(wl.index_keys(0)[None]).cuda(), k8, ks)
    csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, torch.from_numpy(wl.main_kv(0)[None]).cuda(), codes, scales)
    nk = torch.tensor([n], dtype=torch.int32, device="cuda")
    kb, kbs = csa2.coarse_keys(k8, ks, nk, wl.coarse_block)
    q = torch.from_numpy(wl.index_query()).to(torch.bfloat16).cuda()
    w = torch.from_numpy(wl.head_weights()).cuda()
    qa = torch.from_numpy(wl.attn_query()).to(torch.bfloat16).cuda()
    out = torch.empty((1, 1, wl.Hq, wl.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 1, wl.Hq), dtype=torch.float32, device="cuda")

    def step():
        idx = csa2.hier_select(q, w, k8, ks, kb, kbs, nk, wl.coarse_block, wl.coarse_topk, wl.K)
        csa2.sparse_attend(qa, codes, scales, idx, wl.softmax_scale, out=out, lse=lse)

    # one query's step is ~11 short launches: the host's launch rate, not the GPU, would
    # set the pace, so the step is captured once into a HIP graph and replayed
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    # the flat alternative on the same cache: one Full layer (scan all 2^20 keys, Top-1024,
    # attention), also graph-replayed
    layer = dict(mode="full", q_idx=q, w=w, q_attn=qa)
    plan = csa2.GroupPlan([layer], csa2.GroupCache(nk, codes, scales, k8, ks, wl.K, wl.softmax_scale),
                          out_dtype=torch.bfloat16)
    for _ in range(2):
        plan.run()
    torch.cuda.synchronize()
    gflat = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gflat):
        plan.run()
    for _ in range(args.warmup):
        gflat.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        gflat.replay()
    torch.cuda.synchronize()
    flat_ms = (time.perf_counter() - t0) / args.steps * 1e3
    nb = n // wl.coarse_block
    alg = nb * (wl.dk + 4) + wl.coarse_topk * wl.coarse_block * (wl.dk + 4) + wl.K * (wl.D // 2 + 4) + \
        wl.Hq * wl.D * 2 * 2
    # the step's largest kernel is the attention over the 1024 selected entries: its time on
    # a flushed cache (one csa2_sparse_attend call, HIP events) against its bytes (the
    # gathered rows and their indices, the per-channel scales, the query and the output)
    flush = Flusher()
    idx = csa2.hier_select(q, w, k8, ks, kb, kbs, nk, wl.coarse_block, wl.coarse_topk, wl.K)
    att_mean, att_direct, _ = time_cold(
        lambda: csa2.sparse_attend(qa, codes, scales, idx, wl.softmax_scale, out=out, lse=lse), flush, args.score_reps)
    att_bytes = wl.K * (wl.D // 2 + 4) + wl.D * 4 + wl.Hq * wl.D * 2 * 2 + wl.Hq * 4
    att_gbs = att_bytes / (att_mean / 1e3) / 1e9
    res = {
        "metric": "CSA2 decode queries/s at 1M context (two-level indexer)", "value": round(1.0 / (ms_step / 1e3), 1),
        "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": "hier1m: B=1, N=2^20, coarse blocks of 64, top-256 blocks, Top-1024, FP4 E2M1 main KV "
                               "D=512, 64 heads bf16", "global_batch": 1, "seq_len": n, "launch": "hip graph replay"},
        "step_algorithmic_bytes": alg, "flat_full_layer_ms_per_step": round(flat_ms, 5),
        "flat_scan_at_hbm_peak_ms": round(n * (wl.dk + 4) / (HBM_PEAK_GBS * 1e9) * 1e3, 5),
        "roofline": {"bound": "hbm", "achieved": round(att_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(att_gbs / HBM_PEAK_GBS, 5), "traffic": None,
                     "kernel": "sparse attention over the 1024 selected entries: k_attend_part (two splits) + "
                               "k_attend_combine, one csa2_sparse_attend call (cold: flushed before each call; "
                               "latency-bound)", "kernel_ms_mean": round(att_mean, 5),
                     "kernel_ms_direct": round(att_direct, 5), "bytes_per_launch": att_bytes}}
    if not args.no_cpu_baseline:
        import oracle
        kr, ksr = oracle.quantize_fp8(wl.index_keys(0)[None])
        cr, sr = oracle.quantize_fp4(wl.main_kv(0)[None])
        nka = np.array([n], np.int32)
        kbr, kbsr = oracle.coarse_keys(kr, ksr, nka, wl.coarse_block)
        qn, wn, qan = wl.index_query(), wl.head_weights(), wl.attn_query()
        t0 = time.perf_counter()
        ridx, _ = oracle.hier_select(qn, wn, kr, ksr, kbr, kbsr, nka, wl.coarse_block, wl.coarse_topk, wl.K)
        oracle.sparse_attend(qan, cr, sr, ridx, wl.softmax_scale)
        dt = time.perf_counter() - t0
        cb = dict(value=1.0 / dt, unit="queries/s", cores=oracle.num_threads(), kind="oracle",
                  sample="the whole step for the one sequence (coarse scores, top-256 blocks, fine scores, Top-1024, "
                         "attention; coarse keys built beforehand, as on the GPU); %.3f s" % dt)
        cb.update(host_info())
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=3, help="cache copies rotated between steps")
    ap.add_argument("--score-reps", type=int, default=60)
    ap.add_argument("--cpu-seqs", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="group128k",
                    choices=["group128k", "prefill", "full64k", "hier1m", "decoder128k", "group128k_g16",
                             "group128k_swa", "group128k_fp4idx"],
                    help="group128k: the 128K decode group (the headline; default); prefill: the chunked-prefill "
                         "path; full64k: one Full layer at 64K; hier1m: the two-level indexer at 1M; decoder128k: "
                         "the 20-layer decoder schedule at 128K with the candidate pool; group128k_g16: the 128K group with "
                         "the per-16-channel E4M3-scaled FP4 layout; group128k_swa: the 128K group with a 128-token sliding "
                         "window per layer; group128k_fp4idx: the 128K group with the 4-bit indexer")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    ap.add_argument("--stream-probe", type=int, default=0, metavar="BYTES",
                    help="only measure the read-stream ceiling over a buffer of BYTES (flushed before every read) "
                         "and exit")
    ap.add_argument("--cpu-rows", type=int, default=16, help="prefill: new tokens the CPU oracle baseline computes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the CSA2 decode path runs per sequence with no exchange between GPUs, "
              "and the library has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if csa2.device_check() != 0:
        print("not a gfx950 device", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.stream_probe:
        buf = torch.empty(args.stream_probe // 16 * 16, dtype=torch.uint8, device="cuda").fill_(3)
        gbs = stream_ceiling(buf, Flusher())
        print(json.dumps({"stream_probe_bytes": buf.numel(), "read_GBps": round(gbs, 1),
                          "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}), flush=True)
        return
    if args.workload == "prefill":
        run_prefill(args)
        return
    if args.workload == "full64k":
        run_full64k(args)
        return
    if args.workload == "hier1m":
        run_hier1m(args)
        return
    if args.workload == "decoder128k":
        run_decoder128k(args)
        return
    if args.workload == "group128k_g16":
        run_group128k_g16(args)
        return
    if args.workload == "group128k_swa":
        run_group128k_swa(args)
        return
    if args.workload == "group128k_fp4idx":
        run_group128k_fp4idx(args)
        return
    run_group128k(args)


def run_group128k(args):
    wl = workloads.WORKLOADS["group128k"]
    log("building cache (%d copies) ..." % args.copies)
    caches = build_device_cache(wl, args.copies)
    layers = layer_inputs(wl)
    flush = Flusher()
    # headline: flushed, layer by layer
    calls = layer_calls(wl, caches[0], layers)
    log("flushed protocol: warmup %d, timing %d steps" % (args.warmup, args.steps))
    torch.cuda.synchronize()
    ms_step, per_layer, wall = time_flushed(calls, args.steps, args.warmup, flush)
    # the same layers timed by difference (the event pairs' own dispatch cancelled), beside it
    diff_step, diff_layer = time_flushed_by_difference(calls, min(args.steps, 60), flush)
    # warm protocol: the whole group in one call
    plans = [csa2.GroupPlan([dict(L) for L in layers],
                            csa2.GroupCache(c["n_keys"], c["codes"], c["scales"], c["k8"], c["ks"], wl.K,
                                            wl.softmax_scale), out_dtype=torch.bfloat16) for c in caches]
    log("warm protocol: timing %d steps" % args.steps)
    warm_ms = time_warm(plans, args.steps, args.warmup)
    alg = algorithmic_bytes(wl)
    gbs = alg / (ms_step / 1e3) / 1e9
    log("score kernel (cold) and stream ceiling")
    rf = score_roofline(wl, caches[0], layers[0], args.score_reps, flush)
    ceil = stream_ceiling(caches[0]["k8"], flush)
    res = {
        "metric": METRIC, "value": round(wl.B / (ms_step / 1e3), 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": "group128k: Full->Reindex->Reuse decode, B=16, N=131072, indexer 32x64 E4M3, "
                               "Top-512, FP4 E2M1 main KV D=512, 64 heads bf16",
                   "global_batch": wl.B, "seq_len": wl.N, "layers": list(wl.modes),
                   "protocol": "flushed: 512 MiB written before each layer, one C-ABI call per layer, step = sum "
                               "of per-layer HIP-event times"},
        "step_algorithmic_bytes": alg, "step_achieved_GBps": round(gbs, 1),
        "step_pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "step_pct_stream_ceiling": round(100 * gbs / ceil, 2),
        "per_layer_ms": [round(x, 5) for x in per_layer],
        "flushed_loop_wall_s": round(wall, 4),
        "by_difference_ms_per_step": round(diff_step, 5),
        "by_difference_per_layer_ms": [round(x, 5) for x in diff_layer],
        "by_difference_protocol": "flushed, each layer timed by HIP events around (flush, layer) minus events around "
                                  "a flush alone: the event pair's own dispatch cancelled, as in the kernel trace",
        "warm_ms_per_step": round(warm_ms, 5), "warm_value": round(wl.B / (warm_ms / 1e3), 1),
        "warm_protocol": "the group in one csa2_layer_group call (the Full scan keeps its keys for the Reindex "
                         "rescan in the Infinity Cache), %d cache copies rotated between steps" % args.copies,
        "stream_ceiling_GBps": round(ceil, 1),
        "roofline": {"bound": "hbm", "achieved": round(rf["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(rf["achieved"] / HBM_PEAK_GBS, 4), "traffic": counted_traffic(),
                     "frac_of_stream_ceiling": round(rf["achieved"] / ceil, 4),
                     "kernel": "k_score_fp8 (indexer score over every cached key, cold: flushed before each launch)",
                     "kernel_ms_mean": round(rf["kernel_ms_mean"], 5),
                     "kernel_ms_direct": round(rf["kernel_ms_direct"], 5),
                     "kernel_ms_direct_median": round(rf["kernel_ms_direct_median"], 5),
                     "warm_kernel_ms_mean": round(rf["warm_kernel_ms_mean"], 5),
                     "bytes_per_launch": rf["bytes_per_launch"], "traffic_unit": "bytes per launch"},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seqs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
