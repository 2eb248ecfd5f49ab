#!/usr/bin/env python3
"""Benchmark of the MI355X DSA lightning indexer (one GPU).

One step is one layer's indexer pass over the long-prefill workload:
T = 131072 causal tokens, H = 64 indexer heads, d = 128, top-2048, q and k in
OCP FP8 E4M3 with one fp32 scale per token, processed as 32 query chunks of
4096 (chunk c: queries 4096c .. 4096c+4095 against keys 0 .. 4096(c+1)-1).
`value` is its throughput in TFLOP/s (algorithmic flops 2*H*d per scored
query-key pair, 8,590,000,128 pairs per step).  The same line carries the
decode workload (32 sequences x 262144 cached E4M3 keys, bf16 queries,
top-2048) as HBM GB/s, each with its roofline, and the CPU oracle timed on a
bounded sample of the same inputs.

Inputs are generated on the GPU before timing (resident in HBM); outputs,
workspace and streams are allocated before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--adindex [--adindex-len T]] [--dsa16k] [--mtp] [--calib] [--group-query]
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
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer TFLOP/s & Gpairs/s, prefill 128K; decode HBM GB/s at 256K"
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def _pairs_causal(q0, n):
    """Scored pairs of n queries at positions q0..q0+n-1 (each sees t+1 keys)."""
    return n * q0 + n * (n + 1) // 2


def _traffic(*kernel_keys):
    """HBM bytes per launch (summed over the given kernels of one call) from the
    committed rocprofv3 PMC summary, if it was taken on the current kernel
    sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        recs = json.load(open(path))
    except (ValueError, OSError):
        return None
    total = 0.0
    for key in kernel_keys:
        rec = recs.get(key)
        if not rec or rec.get("source_sha1") != _source_sha1(KERNEL_SOURCES[key]):
            return None
        total += rec["hbm_bytes_per_launch"]
    return total


# the sources each measured launch is compiled from, the host code that picks
# its launch shape and top-K mode included (a change to any of them makes the
# committed counters stale)
KERNEL_SOURCES = {
    "dense_topk_fp8_prefill128k": ("dense_topk.hip", "device.h", "launch.h", "api.cpp"),
    "decode_call_decode256k": ("decode.hip", "device.h", "launch.h", "api.cpp"),
}


def _source_sha1(names):
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "sparse_attention_indexer_dsa_amd", "csrc")
    for name in sorted(names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()


def _events_ms(pairs):
    return [s.elapsed_time(e) for s, e in pairs]


# ------------------------------------------------------------------ prefill

def bench_prefill(dsa, args, log):
    from workloads import make_workload
    T, H, d, K, chunk = 131072, 64, 128, 2048, 4096
    log(f"generating prefill inputs T={T} fp8 on the GPU")
    wl = make_workload(3, seed=args.seed, device="cuda")
    q, k, w, qs, ks = wl["q"], wl["k"], wl["w"], wl["q_scale"], wl["k_scale"]
    out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    nchunks = T // chunk
    # one workspace for every chunk: chunks whose rows fit a full-row buffer need more than the last
    ws = torch.empty(max(dsa.workspace_prefill(chunk, (c + 1) * chunk, H, d, K, dsa.DSAIDX_FP8_E4M3)
                         for c in range(nchunks)), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(evs=None):
        for c in range(nchunks):
            q0, q1 = c * chunk, (c + 1) * chunk
            if evs is not None:
                s, e = evs[c]
                s.record(stream)
            dsa.indexer_prefill(q[q0:q1], k[:q1], w[q0:q1], q0, K, qs[q0:q1], ks[:q1], want_score=False,
                                out_idx=out[q0:q1], ws=ws)
            if evs is not None:
                e.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(nchunks)] for _ in range(args.steps)]
    log(f"timing {args.steps} prefill steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = np.array([_events_ms(e) for e in evs])  # [steps, chunks]
    pairs = _pairs_causal(0, T)
    flops = 2 * H * d * pairs
    ms_step = wall * 1e3 / args.steps
    tflops = flops / (ms_step * 1e-3) / 1e12
    # dominant kernel: one streaming score+top-K launch per chunk
    kern_s = launch_ms.sum() * 1e-3 / args.steps
    achieved = flops / kern_s / 1e12
    res = dict(value=tflops, ms_per_step=ms_step, gpairs_per_s=pairs / (ms_step * 1e-3) / 1e9,
               pairs_per_step=pairs, flops_per_step=flops,
               roofline=dict(bound="mfma", kernel="dense_topk_kernel<fp8>", achieved=achieved,
                             peak=PEAK_FP8_TFLOPS, unit="TFLOP/s", frac=achieved / PEAK_FP8_TFLOPS,
                             launches_per_step=nchunks,
                             avg_launch_ms=float(launch_ms.mean()),
                             flops_per_launch=flops / nchunks,
                             traffic=_traffic("dense_topk_fp8_prefill128k")))
    cpu = None
    if not args.no_cpu:
        cpu = cpu_prefill(wl, out, args, log)
    return res, cpu


def cpu_prefill(wl, out, args, log):
    """The oracle on a stratified sample of query rows of the same workload;
    the sampled GPU rows are checked against it (tolerance rule)."""
    import oracle
    from tests.parity import compare
    T, K = 131072, 2048
    n = args.cpu_rows
    rows = np.unique(np.concatenate([np.linspace(0, T - 1, n - 2).astype(np.int64), [T - 2, T - 1]]))
    log(f"cpu oracle on {len(rows)} sampled prefill rows")
    qh = wl["q"].cpu()
    kh, wh = wl["k"].cpu(), wl["w"].cpu()
    qsh, ksh = wl["q_scale"].cpu(), wl["k_scale"].cpu()
    t0 = time.perf_counter()
    ri, rs = oracle.prefill(qh, kh, wh, "fp8", 0, K, qsh, ksh, rows=rows)
    dt = time.perf_counter() - t0
    pairs = int((rows + 1).sum())
    gi = out[torch.as_tensor(rows, device="cuda")].cpu().numpy()

    def score_of(r, keys):
        return oracle.score_pairs(qh, kh, wh, np.full(len(keys), rows[r]), keys, "fp8", "fp8", qsh, ksh)
    parity = "ok"
    try:
        compare(gi, None, ri, rs, False, score_of)
    except AssertionError as e:  # reported, not raised: the bench still prints its line
        parity = "FAILED: " + str(e)[:300]
    return dict(value=2 * 64 * 128 * pairs / dt / 1e12, unit="TFLOP/s", gpairs_per_s=pairs / dt / 1e9,
                cores=oracle.max_threads(), kind="oracle", seconds=dt,
                sample=f"{len(rows)} query rows of the 128K prefill spread over positions 0..{T - 1} "
                       f"({pairs} scored pairs), fp64 C oracle with OpenMP over rows",
                parity_of_sampled_gpu_rows=parity)


# ------------------------------------------------------------------- decode

def bench_decode(dsa, args, log):
    from workloads import make_workload
    B, N, H, d, K = 32, 262144, 64, 128, 2048
    log(f"generating decode inputs B={B} N={N} on the GPU")
    wl = make_workload(4, seed=args.seed, device="cuda")
    t = wl.tensors
    out = torch.empty((B, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.workspace_decode(B, N, H, d, K), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        dsa.indexer_decode(t["q"], t["k_cache"], t["k_scale"], t["w"], t["seq_lens"], K, want_score=False,
                           out_idx=out, ws=ws)

    for _ in range(max(args.warmup, 1) * 3):
        step()
    torch.cuda.synchronize()
    nsteps = args.steps * 20  # a decode step is ~0.2 ms: time many
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsteps)]
    log(f"timing {nsteps} decode steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in evs:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = np.array(_events_ms(evs))
    alg_bytes = B * N * d + B * N * 4 + B * H * d * 2 + B * H * 4 + B * K * 4
    ms_step = wall * 1e3 / nsteps
    gbs = alg_bytes / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes / (call_ms.mean() * 1e-3) / 1e9
    res = dict(workload="decode scan: 32 sequences x 262144 cached keys, E4M3 cache + fp32 per-token scale, "
                        "bf16 query, H=64, d=128, top-2048",
               value=gbs, unit="GB/s", ms_per_step=ms_step, steps=nsteps,
               gpairs_per_s=B * N / (ms_step * 1e-3) / 1e9, bytes_per_step=alg_bytes,
               roofline=dict(bound="hbm", kernel="fill + decode_scan + decode_classify + decode_select + decode_emit (one call)",
                             achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s", frac=achieved / PEAK_HBM_GBS,
                             avg_launch_ms=float(call_ms.mean()), bytes_per_launch=alg_bytes,
                             traffic=_traffic("decode_call_decode256k")))
    if not args.no_cpu:
        import oracle
        from tests.parity import compare
        rows = np.arange(0, B, max(1, B // args.cpu_decode_rows))[:args.cpu_decode_rows]
        log(f"cpu oracle on {len(rows)} decode rows")
        h = {k2: v.cpu() for k2, v in t.items()}
        t0 = time.perf_counter()
        ri, rs = oracle.decode(h["q"], h["k_cache"], h["k_scale"], h["w"], h["seq_lens"], K, rows=rows)
        dt = time.perf_counter() - t0
        kc = h["k_cache"].reshape(B * N, d)
        ksc = h["k_scale"].reshape(B * N)

        def score_of(r, keys):
            return oracle.score_pairs(h["q"], kc, h["w"], np.full(len(keys), rows[r]), rows[r] * N + keys,
                                      "bf16", "fp8", None, ksc)
        parity = "ok"
        try:
            compare(out.cpu().numpy()[rows], None, ri, rs, False, score_of)
        except AssertionError as e:
            parity = "FAILED: " + str(e)[:300]
        per_row = alg_bytes / B
        res["cpu_baseline"] = dict(value=per_row * len(rows) / dt / 1e9, unit="GB/s",
                                   gpairs_per_s=len(rows) * N / dt / 1e9, cores=oracle.max_threads(),
                                   kind="oracle", seconds=dt,
                                   sample=f"{len(rows)} of the 32 decode rows (full 262144-key scans)",
                                   parity_of_sampled_gpu_rows=parity)
    return res


# ------------------------------------------------------------------ ADIndex

def bench_adindex(dsa, args, log):
    from workloads import make_workload
    T, H, d, K, G, P = args.adindex_len, 64, 128, 2048, 16, 8192
    log(f"generating ADIndex inputs T={T} bf16 on the GPU")
    wl = make_workload(5, seed=args.seed, device="cuda", T=T)
    t = wl.tensors
    out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    out_pool = torch.empty((T, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.workspace_group_bank(T, T, H, H, d, G, P, K, dsa.DSAIDX_BF16, dsa.POOL_MEAN),
                     dtype=torch.uint8, device="cuda")
    dense_out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    wsd = torch.empty(dsa.workspace_prefill(T, T, H, d, K, dsa.DSAIDX_BF16), dtype=torch.uint8, device="cuda")

    def step():
        dsa.indexer_group_bank(t["q"], t["k"], t["w"], t["qbar"], t["wbar"], 0, G, P, K, want_score=False,
                               out_idx=out, ws=ws)

    def step_pool():
        dsa.indexer_group_bank(t["q"], t["k"], t["w"], None, None, 0, G, P, K, flags=dsa.POOL_MEAN,
                               want_score=False, out_idx=out_pool, ws=ws)

    def dense():
        dsa.indexer_prefill(t["q"], t["k"], t["w"], 0, K, want_score=False, out_idx=dense_out, ws=wsd)

    res = {}
    for name, fn, steps in (("adindex", step, args.steps), ("adindex_pool", step_pool, args.steps),
                            ("dense", dense, max(1, args.steps // 2))):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) * 1e3 / steps
    pairs = dsa.indexer_group_bank_pairs(T, 0, G, P)
    flops = 2 * H * d * pairs
    dense_pairs = _pairs_causal(0, T)
    # recall of the bank result against the dense top-K (coverage of Section 5)
    sample = torch.arange(8192, T, 997, device="cuda")
    b = dense_out[sample].cpu().numpy()

    def recall(o):
        return float(np.mean([len(np.intersect1d(x, y)) / len(y) for x, y in zip(o[sample].cpu().numpy(), b)]))
    rec, rec_pool = recall(out), recall(out_pool)
    return dict(workload=f"ADIndex group token bank: T={T}, G=16, P=8192, H=Hs=64, d=128, top-2048, bf16",
                ms_per_step=res["adindex"], tflops=flops / (res["adindex"] * 1e-3) / 1e12,
                gpairs_per_s=pairs / (res["adindex"] * 1e-3) / 1e9, pairs=pairs,
                dense_ms=res["dense"], dense_tflops=2 * H * d * dense_pairs / (res["dense"] * 1e-3) / 1e12,
                speedup_vs_dense=res["dense"] / res["adindex"], scoring_count_ratio=dense_pairs / pairs,
                recall_vs_dense=rec,
                pooled=dict(ms_per_step=res["adindex_pool"], speedup_vs_dense=res["dense"] / res["adindex_pool"],
                            recall_vs_dense=rec_pool,
                            note="training-free group query: mean of the group's own queries and gates"),
                recall_note="synthetic i.i.d. queries: recall reflects the random inputs, not trained data",
                roofline=dict(bound="mfma", achieved=flops / (res["adindex"] * 1e-3) / 1e12,
                              peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=flops / (res["adindex"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS))


# ---------------------------------------------------- DSA-shaped bf16 prefill

def bench_dsa16k(dsa, args, log):
    """One layer of DSA-shaped bf16 prefill: T=16384, H=64, d=128, top-2048, one
    call (134,225,920 pairs, 2.199 TFLOP)."""
    from workloads import make_workload
    T, H, d, K = 16384, 64, 128, 2048
    log("generating DSA bf16 prefill inputs T=16384 on the GPU")
    wl = make_workload(2, seed=args.seed, device="cuda")
    t = wl.tensors
    out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.workspace_prefill(T, T, H, d, K, dsa.DSAIDX_BF16), dtype=torch.uint8, device="cuda")

    def step():
        dsa.indexer_prefill(t["q"], t["k"], t["w"], 0, K, want_score=False, out_idx=out, ws=ws)
    step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    pairs = _pairs_causal(0, T)
    tf = 2 * H * d * pairs / (ms * 1e-3) / 1e12
    return dict(workload="DSA prefill, one layer: T=16384, H=64, d=128, top-2048, bf16", ms_per_call=ms,
                tflops=tf, gpairs_per_s=pairs / (ms * 1e-3) / 1e9, frac_of_bf16_peak=tf / PEAK_BF16_TFLOPS)


# ------------------------------------------------------------------ MTP

def bench_mtp(dsa, args, log):
    """MTP target verification at 256K (the pages' decode-indexer speedups are
    quoted at 256K for 16-query windows and (G, P) in {8, 16} x {8K, 16K}).
    The group indexer has 8 heads (one eighth of the 64 indexer heads)."""
    from workloads import make_mtp
    B, N, m, H, Hs, d, K = 8, 262144, 16, 64, 8, 128, 2048
    out = torch.empty((B, m, K), dtype=torch.int32, device="cuda")
    dense_out = torch.empty_like(out)
    res = dict(workload=f"MTP verification: B={B} sequences x {m}-query windows, the last query seeing all "
                        f"{N} keys of an E4M3 cache, H=64, Hs={Hs}, d=128, top-{K}", configs=[])
    wl = None
    for G, P in ((8, 8192), (16, 8192), (8, 16384), (16, 16384)):
        if wl is None or wl.params["G"] != G:
            log(f"generating MTP inputs (G={G}) on the GPU")
            wl = make_mtp(B=B, N=N, m=m, H=H, Hs=Hs, d=d, topk=K, G=G, P=P, dist="normal", seed=args.seed,
                          device="cuda")
        t = wl.tensors
        ws = torch.empty(dsa.workspace_mtp(B, N, m, H, Hs, d, G, P, K), dtype=torch.uint8, device="cuda")

        def step():
            dsa.indexer_mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], t["qbar"], t["wbar"], t["prefix_lens"], G,
                            P, K, want_score=False, out_idx=out, ws=ws)

        def dense():
            dsa.indexer_mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], None, None, t["prefix_lens"], G, P, K,
                            flags=dsa.NO_BANK, want_score=False, out_idx=dense_out, ws=ws)
        ms = {}
        for name, fn in (("mtp", step), ("dense", dense)):
            fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            ms[name] = (time.perf_counter() - t0) * 1e3 / args.steps
        lens = t["prefix_lens"].cpu().numpy()
        pairs = dsa.indexer_mtp_pairs(lens, N, m, G, P)
        dense_pairs = dsa.indexer_mtp_pairs(lens, N, m, G, P, dsa.NO_BANK)
        a, b = out.reshape(B * m, K).cpu().numpy(), dense_out.reshape(B * m, K).cpu().numpy()
        rec = float(np.mean([len(np.intersect1d(x, y)) / len(y) for x, y in zip(a, b)]))
        # one read of every sequence's cache and scales is the least any scan needs
        cache_bytes = B * N * (d + 4)
        res["configs"].append(dict(G=G, P=P, ms_per_call=ms["mtp"], dense_ms=ms["dense"],
                                   speedup_vs_dense=ms["dense"] / ms["mtp"],
                                   scoring_count_ratio=dense_pairs / pairs, pairs=pairs,
                                   cache_read_gbs=cache_bytes / (ms["mtp"] * 1e-3) / 1e9,
                                   dense_cache_read_gbs=cache_bytes / (ms["dense"] * 1e-3) / 1e9,
                                   recall_vs_dense=rec))
        log(f"MTP G={G} P={P}: {ms['mtp']:.3f} ms, dense {ms['dense']:.3f} ms")
    res["recall_note"] = "synthetic i.i.d. queries and a random group query: recall is not a quality figure"
    return res


# ------------------------------------------------------------ group query

def bench_group_query(dsa, args, log):
    """Eq. (6)-(7) for the 64K ADIndex layer: G = 16 (4096 groups), DeepSeek-
    like latent sizes (dc = 1536 query latent, dh = 7168 hidden), Hs = 8 heads
    of d = 128.  HBM-bound: the latents and hidden states are read once."""
    T, dc, dh, Hs, d, G = 65536, 1536, 7168, 8, 128, 16
    log("generating group-query inputs on the GPU")
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed)
    c = torch.randn(T, dc, generator=g, device="cuda").to(torch.bfloat16)
    h = torch.randn(T, dh, generator=g, device="cuda").to(torch.bfloat16)
    wp = (torch.randn(dc, 3 * dc, generator=g, device="cuda") / (3 * dc) ** 0.5).to(torch.bfloat16)
    wq = (torch.randn(Hs * d, dc, generator=g, device="cuda") / dc ** 0.5).to(torch.bfloat16)
    wg = (torch.randn(Hs, dh, generator=g, device="cuda") / dh ** 0.5).to(torch.bfloat16)
    ws = torch.empty(dsa.lib().indexer_group_query_workspace_size(T, dc, dh, Hs, d, G), dtype=torch.uint8,
                     device="cuda")
    qb = torch.empty((T // G, Hs, d), dtype=torch.bfloat16, device="cuda")
    wb = torch.empty((T // G, Hs), dtype=torch.float32, device="cuda")

    def step():
        dsa.indexer_group_query(c, h, wp, wq, wg, G, Hs, d, 0, 64, qbar=qb, wbar=wb, ws=ws)
    step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    nbytes = T * (dc + dh) * 2
    n = T // G
    flops = 2 * n * (3 * dc * dc + dc * Hs * d + dh * Hs)
    return dict(workload=f"group query (Eq. 6-7): T={T}, G={G}, dc={dc}, dh={dh}, Hs={Hs}, d={d}, bf16",
                ms_per_call=ms, input_read_gbs=nbytes / (ms * 1e-3) / 1e9,
                frac_of_hbm=nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                product_tflops_over_call=flops / (ms * 1e-3) / 1e12,
                note="product flops over the whole call, which the HBM-bound pooling read dominates")


# ------------------------------------------------------------ calibration

def bench_calib(dsa, args, log):
    """Calibration statistics over a 128K-token layer's reference top-2048 sets:
    Eq. (4) union sizes for G = 4, 8, 16 and per-row overlaps.  HBM-bound: one
    read of the [T, K] int32 index sets (two for the overlap)."""
    T, K = 131072, 2048
    log("generating sorted index sets [131072, 2048] on the GPU")
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed)
    idx = torch.randint(0, T, (T, K), generator=g, device="cuda", dtype=torch.int32).sort(dim=1).values
    other = idx.roll(1, 0).contiguous()
    res = dict(workload=f"calibration statistics: index sets [{T}, {K}] int32", runs=[])
    bytes_once = T * K * 4
    for name, fn, nbytes in ([(f"union_sizes G={G}", (lambda G=G: dsa.union_sizes(idx, G)), bytes_once)
                              for G in (4, 8, 16)] + [("topk_overlap", lambda: dsa.topk_overlap(idx, other),
                                                       2 * bytes_once)]):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        res["runs"].append(dict(name=name, ms=ms, gbs=nbytes / (ms * 1e-3) / 1e9,
                                frac_of_hbm=nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS))
        log(f"{name}: {ms:.3f} ms")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--cpu-decode-rows", type=int, default=32)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--adindex", action="store_true", help="also time the ADIndex group-bank workload")
    ap.add_argument("--adindex-len", type=int, default=65536, metavar="T",
                    help="sequence length of the ADIndex workload (65536; the pages quote 262144)")
    ap.add_argument("--mtp", action="store_true", help="also time MTP verification windows at 256K")
    ap.add_argument("--dsa16k", action="store_true", help="also time the 16K bf16 DSA prefill layer")
    ap.add_argument("--calib", action="store_true", help="also time the calibration statistics kernels")
    ap.add_argument("--group-query", action="store_true", help="also time the group query construction")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES device-to-device 5 times (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.copy_probe:
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "copies": 5}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the indexer path here runs on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import sparse_attention_indexer_dsa_amd as dsa
    dsa.lib()

    pre, cpu = bench_prefill(dsa, args, log)
    line = {
        "metric": METRIC,
        "value": pre["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "long prefill, one layer: T=131072, H_I=64, d=128, top-2048, E4M3 q and k "
                               "with per-token fp32 scales, w fp32, 32 causal query chunks of 4096",
                   "T": 131072, "H": 64, "d": 128, "topk": 2048, "chunk": 4096, "seed": args.seed},
        "gpairs_per_s": pre["gpairs_per_s"],
        "pairs_per_step": pre["pairs_per_step"],
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
    }
    if not args.no_decode:
        line["decode"] = bench_decode(dsa, args, log)
    if args.adindex:
        line["adindex"] = bench_adindex(dsa, args, log)
    if args.dsa16k:
        line["dsa16k"] = bench_dsa16k(dsa, args, log)
    if args.mtp:
        line["mtp"] = bench_mtp(dsa, args, log)
    if args.calib:
        line["calib"] = bench_calib(dsa, args, log)
    if args.group_query:
        line["group_query"] = bench_group_query(dsa, args, log)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
