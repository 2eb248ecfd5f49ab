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

The line also carries, each with its roofline and an oracle baseline on
sampled rows: the 16K bf16 DSA prefill layer (dsa16k), the 64K ADIndex group
bank against the dense indexer (adindex), the 61-layer pass with Table 9's
per-layer (G, P) (layerwise), and the plain HBM read stream (decode.read_ceiling).
If any sampled GPU rows disagree with the oracle, `value` is null, the line
says why, and the exit status is 1.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-dsa16k] [--no-adindex]
                    [--adindex-len T] [--no-layerwise] [--mtp] [--calib] [--group-query]
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


def _cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_fields(oracle):
    return dict(cores=oracle.max_threads(), cpu_model=_cpu_model(), host_logical_cpus=os.cpu_count())


PARITY = {}  # leg name -> "ok" or the failure message; any failure invalidates the line


def _parity(name, fn):
    """Run a parity check of sampled GPU rows against the oracle; record it."""
    try:
        fn()
        PARITY[name] = "ok"
    except AssertionError as e:
        PARITY[name] = "FAILED: " + str(e)[:300]
    return PARITY[name]


def _stratified(T, n, always=()):
    """n rows spread evenly over 0..T-1, the last 16 rows and `always`."""
    r = np.concatenate([np.linspace(0, T - 1, n).astype(np.int64), np.arange(T - 16, T),
                        np.asarray(always, np.int64)])
    return np.unique(r[(r >= 0) & (r < T)])


def _timed_calls(fn, steps, stream):
    """Time `steps` calls of fn with HIP events on `stream` (after one warm
    call); returns (wall ms per call, event ms per call)."""
    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for s_, e_ in evs:
        s_.record(stream)
        fn()
        e_.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, float(np.mean(_events_ms(evs)))


# ------------------------------------------------------------------ prefill

def bench_prefill(dsa, args, log):
    from workloads import make_workload
    T, H, d, K, chunk = 131072, 64, 128, 2048, 4096
    log(f"generating prefill inputs T={T} fp8 on the GPU")
    wl = make_workload(3, seed=args.seed, device="cuda")
    q, k, w, qs, ks = wl["q"], wl["k"], wl["w"], wl["q_scale"], wl["k_scale"]
    out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    nchunks = T // chunk
    # one workspace serves every chunk (its size does not depend on the key count)
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
    # the sustained matrix-core stream, right after the prefill (same clocks
    # and temperature)
    res["mfma_ceiling"] = bench_mfma_probe(dsa, log)
    res["mfma_ceiling"]["dense_frac_of_ceiling"] = achieved / res["mfma_ceiling"]["tflops"]
    cpu = None
    if not args.no_cpu:
        cpu = cpu_prefill(wl, out, args, log)
    return res, cpu


def bench_mfma_probe(dsa, log):
    """The matrix-core stream (indexer_mfma_probe: back-to-back 32x32x64 E4M3
    MFMAs on register operands, four accumulators per wave, one workgroup per
    CU) at 1, 2 and 4 waves per SIMD, timed with HIP events, for two operand
    distributions: bytes spanning the whole E4M3 range with random signs (like
    the prefill's E4M3 q and k) and small positive magnitudes; and the same
    stream of 32x32x16 bf16 MFMAs on random signs and mantissas (the bf16
    paths' ceiling).  The chip's
    power limit makes the sustained rate depend on the data; the best rate on
    whole-range operands is the ceiling the fp8 prefill kernel is compared
    with.  Each wave's shader-clock and 100 MHz constant-clock counts give the
    clock it ran at."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    log(f"timing the E4M3 MFMA stream on {ncu} CUs")

    def sweep(mask, dtype="fp8"):
        by_wps = {}
        kdim = 64 if dtype == "fp8" else 16  # k of one MFMA: 32x32x64 E4M3, 32x32x16 bf16
        for wps in (1, 2, 4):
            iters = (24576 if dtype == "fp8" else 49152) // wps
            out, clocks = dsa.mfma_probe(iters, wps, ncu, mask, dtype=dtype)
            _, ms = _timed_calls(lambda: dsa.mfma_probe(iters, wps, ncu, mask, out, clocks, dtype=dtype), 20, stream)
            flops = 2.0 * 32 * 32 * kdim * 4 * iters * (ncu * 4 * wps)
            c = clocks.cpu().numpy().astype(np.float64)
            mhz = float(np.mean(c[:, 0] / (c[:, 1] / 100.0)))  # counts per microsecond
            by_wps[wps] = dict(tflops=flops / (ms * 1e-3) / 1e12, ms=ms, shader_clock_mhz=mhz)
        best = max(by_wps, key=lambda k: by_wps[k]["tflops"])
        return by_wps[best]["tflops"], best, {str(k): {kk: round(vv, 3) for kk, vv in v.items()}
                                              for k, v in by_wps.items()}

    tf, best, by = sweep(0xFEFEFEFE)
    tf_low, best_low, by_low = sweep(0x37373737)
    tf_bf, best_bf, by_bf = sweep(0xBFFFBFFF, "bf16")
    return dict(kernel="mfma_probe_kernel (indexer_mfma_probe)", operands="whole E4M3 range, random signs "
                "(operand_mask 0xFEFEFEFE)", tflops=tf, frac_of_peak=tf / PEAK_FP8_TFLOPS, best_waves_per_simd=best,
                by_waves_per_simd=by,
                small_operands=dict(operands="magnitudes below 1, positive (operand_mask 0x37373737)", tflops=tf_low,
                                    frac_of_peak=tf_low / PEAK_FP8_TFLOPS, best_waves_per_simd=best_low,
                                    by_waves_per_simd=by_low),
                bf16=dict(kernel="mfma_probe_kernel, 32x32x16 bf16", operands="random signs and mantissas, "
                          "magnitudes below 2 (operand_mask 0xBFFFBFFF)", tflops=tf_bf,
                          frac_of_peak=tf_bf / PEAK_BF16_TFLOPS, best_waves_per_simd=best_bf,
                          by_waves_per_simd=by_bf))


def cpu_prefill(wl, out, args, log):
    """The oracle on a stratified sample of query rows of the same workload;
    the sampled GPU rows are checked against it (tolerance rule)."""
    import oracle
    from tests.parity import compare, pair_refs
    T, K = 131072, 2048
    rows = _stratified(T, args.cpu_rows)
    log(f"cpu oracle on {len(rows)} sampled prefill rows")
    qh = wl["q"].cpu()
    kh, wh = wl["k"].cpu(), wl["w"].cpu()
    qsh, ksh = wl["q_scale"].cpu(), wl["k_scale"].cpu()
    t0 = time.perf_counter()
    ri, rs = oracle.prefill(qh, kh, wh, "fp8", 0, K, qsh, ksh, rows=rows)
    dt = time.perf_counter() - t0
    pairs = int((rows + 1).sum())
    gi = out[torch.as_tensor(rows, device="cuda")].cpu().numpy()

    score_of, cond_of = pair_refs(qh, kh, wh, rows, "fp8", "fp8", qsh, ksh)
    parity = _parity("prefill128k", lambda: compare(gi, None, ri, rs, False, score_of, ref_cond_of=cond_of))
    return dict(value=2 * 64 * 128 * pairs / dt / 1e12, unit="TFLOP/s", gpairs_per_s=pairs / dt / 1e9,
                kind="oracle", seconds=dt, **_cpu_fields(oracle),
                sample=f"{len(rows)} query rows of the 128K prefill: evenly spread over positions 0..{T - 1} "
                       f"and the last 16 ({pairs} scored pairs), fp64 C oracle with OpenMP over rows",
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
        from tests.parity import compare, pair_refs
        rows = np.arange(0, B, max(1, B // args.cpu_decode_rows))[:args.cpu_decode_rows]
        log(f"cpu oracle on {len(rows)} decode rows")
        h = {k2: v.cpu() for k2, v in t.items()}
        t0 = time.perf_counter()
        ri, rs = oracle.decode(h["q"], h["k_cache"], h["k_scale"], h["w"], h["seq_lens"], K, rows=rows)
        dt = time.perf_counter() - t0
        kc = h["k_cache"].reshape(B * N, d)
        ksc = h["k_scale"].reshape(B * N)

        score_of, cond_of = pair_refs(h["q"], kc, h["w"], rows, "bf16", "fp8", None, ksc,
                                      key_of=lambda r, keys: rows[r] * N + keys)
        parity = _parity("decode256k", lambda: compare(out.cpu().numpy()[rows], None, ri, rs, False, score_of,
                                                       ref_cond_of=cond_of))
        per_row = alg_bytes / B
        res["cpu_baseline"] = dict(value=per_row * len(rows) / dt / 1e9, unit="GB/s",
                                   gpairs_per_s=len(rows) * N / dt / 1e9, kind="oracle", seconds=dt,
                                   **_cpu_fields(oracle),
                                   sample=f"{len(rows)} of the 32 decode rows (full 262144-key scans)",
                                   parity_of_sampled_gpu_rows=parity)
    del t, wl
    res["read_ceiling"] = bench_read_probe(dsa, args, log)
    res["read_ceiling"]["decode_frac_of_ceiling"] = achieved / res["read_ceiling"]["gbs"]
    return res


# workgroup counts the read probe is timed at: the rate of a grid-stride
# read depends on the grid (how the concurrent addresses fall on the HBM
# channels), so the ceiling is the best of several
READ_PROBE_GRIDS = (256, 512, 2048, 8192, 16384, 32768)


def bench_read_probe(dsa, args, log):
    """The plain HBM read stream (indexer_read_probe: every byte of a 4 GiB
    buffer read once with coalesced 16-byte loads), timed with HIP events at
    several grid sizes: the best is the practical ceiling the memory-bound
    decode scan is compared with."""
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    out = torch.empty(max(READ_PROBE_GRIDS), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    log(f"timing the plain read stream (4 GiB) at grids {READ_PROBE_GRIDS}")
    by_grid = {}
    for g in READ_PROBE_GRIDS:
        _, ms = _timed_calls(lambda: dsa.read_probe(buf, g, out), 10, stream)
        by_grid[g] = nbytes / (ms * 1e-3) / 1e9
    best = max(by_grid, key=by_grid.get)
    gbs = by_grid[best]
    return dict(kernel="read_probe_kernel (indexer_read_probe)", bytes=nbytes,
                ms=nbytes / (gbs * 1e9) * 1e3, gbs=gbs, frac_of_peak=gbs / PEAK_HBM_GBS, best_grid=best,
                gbs_by_grid={str(k): round(v, 1) for k, v in by_grid.items()})


# ------------------------------------------------------------------ ADIndex

def bench_adindex(dsa, args, log):
    """The ADIndex group token bank (T=65536, G=16, P=8192, H=Hs=64, d=128,
    bf16) against the dense bf16 indexer at the same length; the roofline is
    the method's algorithmic flops (2*H*d per scored pair) over the event-timed
    call, against the bf16 MFMA peak."""
    from workloads import make_workload
    T, H, d, K, G, P = args.adindex_len, 64, 128, 2048, 16, 8192
    log(f"generating ADIndex inputs T={T} bf16 on the GPU")
    wl = make_workload(5, seed=args.seed, device="cuda", T=T)
    t = wl.tensors
    out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    out_pool = torch.empty((T, K), dtype=torch.int32, device="cuda")
    bank = torch.empty((-(-T // G), P), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.workspace_group_bank(T, T, H, H, d, G, P, K, dsa.DSAIDX_BF16, dsa.POOL_MEAN),
                     dtype=torch.uint8, device="cuda")
    dense_out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    wsd = torch.empty(dsa.workspace_prefill(T, T, H, d, K, dsa.DSAIDX_BF16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        dsa.indexer_group_bank(t["q"], t["k"], t["w"], t["qbar"], t["wbar"], 0, G, P, K, want_score=False,
                               out_idx=out, out_bank=bank, ws=ws)

    def step_pool():
        dsa.indexer_group_bank(t["q"], t["k"], t["w"], None, None, 0, G, P, K, flags=dsa.POOL_MEAN,
                               want_score=False, out_idx=out_pool, ws=ws)

    def dense():
        dsa.indexer_prefill(t["q"], t["k"], t["w"], 0, K, want_score=False, out_idx=dense_out, ws=wsd)

    log("timing the ADIndex bank path, its pooled variant and the dense indexer")
    ms, ev = {}, {}
    for name, fn, steps in (("adindex", step, args.steps), ("adindex_pool", step_pool, args.steps),
                            ("dense", dense, max(2, args.steps // 2))):
        ms[name], ev[name] = _timed_calls(fn, steps, stream)
    # the other (G, P) settings of Eq. (5)'s search, with the training-free
    # pooled group query (the q-bar input above is G = 16's); G = 4 refines in
    # the general kernel, G = 8 and 16 in the dense kernel's gather mode
    settings = []
    for g2, p2 in ((4, 8192), (8, 8192), (16, 8192), (8, 16384), (16, 16384)):
        ws2 = torch.empty(dsa.workspace_group_bank(T, T, H, H, d, g2, p2, K, dsa.DSAIDX_BF16, dsa.POOL_MEAN),
                          dtype=torch.uint8, device="cuda")
        fn = (lambda g2=g2, p2=p2, ws2=ws2: dsa.indexer_group_bank(
            t["q"], t["k"], t["w"], None, None, 0, g2, p2, K, flags=dsa.POOL_MEAN, want_score=False,
            out_idx=out_pool, ws=ws2))
        m2, _ = _timed_calls(fn, max(2, args.steps // 2), stream)
        pr = dsa.indexer_group_bank_pairs(T, 0, g2, p2)
        settings.append(dict(G=g2, P=p2, ms_per_call=m2, speedup_vs_dense=ms["dense"] / m2,
                             scoring_count_ratio=_pairs_causal(0, T) / pr,
                             tflops=2 * H * d * pr / (m2 * 1e-3) / 1e12))
        del ws2
    step()  # leave the bank result (and its banks) in `out` for the parity leg
    torch.cuda.synchronize()
    pairs = dsa.indexer_group_bank_pairs(T, 0, G, P)
    flops = 2 * H * d * pairs
    dense_pairs = _pairs_causal(0, T)
    # recall of the bank result against the dense top-K (coverage of Section 5)
    sample = torch.arange(8192, T, 997, device="cuda")
    b = dense_out[sample].cpu().numpy()

    def recall(o):
        return float(np.mean([len(np.intersect1d(x, y)) / len(y) for x, y in zip(o[sample].cpu().numpy(), b)]))
    rec, rec_pool = recall(out), recall(out_pool)
    achieved = flops / (ev["adindex"] * 1e-3) / 1e12
    res = dict(workload=f"ADIndex group token bank: T={T}, G=16, P=8192, H=Hs=64, d=128, top-2048, bf16",
               ms_per_step=ms["adindex"], tflops=flops / (ms["adindex"] * 1e-3) / 1e12,
               gpairs_per_s=pairs / (ms["adindex"] * 1e-3) / 1e9, pairs=pairs,
               dense_ms=ms["dense"], dense_tflops=2 * H * d * dense_pairs / (ms["dense"] * 1e-3) / 1e12,
               speedup_vs_dense=ms["dense"] / ms["adindex"], scoring_count_ratio=dense_pairs / pairs,
               recall_vs_dense=rec,
               pooled=dict(ms_per_step=ms["adindex_pool"], speedup_vs_dense=ms["dense"] / ms["adindex_pool"],
                           recall_vs_dense=rec_pool,
                           note="training-free group query: mean of the group's own queries and gates"),
               recall_note="synthetic i.i.d. queries: recall reflects the random inputs, not trained data",
               pooled_settings=settings,
               roofline=dict(bound="mfma", kernel="indexer_group_bank (group scan + refinement + fallback "
                                                  "launches of dense_topk_kernel<bf16>, one call)",
                             achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                             frac=achieved / PEAK_BF16_TFLOPS, avg_launch_ms=ev["adindex"],
                             flops_per_launch=flops, traffic=None))
    if T == 65536 and not args.no_cpu:
        res["cpu_baseline"] = cpu_adindex(wl, out, bank, G, P, K, args, log)
    res["_dense_ms"] = ms["dense"]
    return res


def cpu_adindex(wl, out, bank, G, P, K, args, log):
    """The oracle's group bank on stratified query rows (the last 16 and the
    groups around the fallback/bank boundary included); the sampled GPU rows
    and their groups' banks are checked against it under the tolerance rule."""
    import oracle
    from tests.parity import compare, pair_refs, refine_over_bank
    T = wl.params["T"]
    rows = _stratified(T, args.cpu_adindex_rows, always=np.arange(8176, 8208))
    log(f"cpu oracle on {len(rows)} sampled ADIndex rows")
    h = {k: v.cpu() for k, v in wl.tensors.items()}
    t0 = time.perf_counter()
    ri, rs, rb, _ = oracle.group_bank(h["q"], h["k"], h["w"], h["qbar"], h["wbar"], "bf16", 0, G, P, K,
                                      rows=rows, want_bank=True)
    dt = time.perf_counter() - t0
    gi = out[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    gbank = bank.cpu().numpy()
    groups = np.unique(rows // G)
    # scored pairs of the sample: each sampled group's anchor scan (once) and
    # each sampled row's candidates
    pairs = 0
    for g in groups:
        a = g * G
        pairs += (a + 1) if a + 1 > P else 0
    for r in rows:
        a = (r // G) * G
        pairs += (r + 1) if a + 1 <= P else min(P, a + 1) + (r - a)

    def check():
        score_of, cond_of = pair_refs(h["q"], h["k"], h["w"], rows, "bf16", "bf16")
        for g in groups:
            if (rb[g] == -1).all():
                assert (gbank[g] == -1).all(), f"bank {g} should be empty"
                continue
            bank_score, bank_cond = pair_refs(h["qbar"], h["k"], h["wbar"], [g], "bf16", "bf16")
            v = rb[g][rb[g] >= 0]
            compare(gbank[g:g + 1], None, rb[g:g + 1], bank_score(0, v)[None, :], False, bank_score,
                    label=f"bank {g}", ref_cond_of=bank_cond)
        same = np.array([np.array_equal(rb[r // G], gbank[r // G]) for r in rows])
        sel = np.nonzero(same)[0]
        compare(gi[sel], None, ri[sel], rs[sel], False, lambda r, keys: score_of(sel[r], keys),
                ref_cond_of=lambda r, keys: cond_of(sel[r], keys))
        other = rows[~same]
        if len(other):  # groups whose bank differs by tolerated swaps: Eq. (14) over the GPU's bank
            oi, osc = refine_over_bank(h, gbank, other, G, K)
            o_score, o_cond = pair_refs(h["q"], h["k"], h["w"], other, "bf16", "bf16")
            compare(gi[~same], None, oi, osc, False, o_score, label="own bank", ref_cond_of=o_cond)
    parity = _parity("adindex64k", check)
    return dict(value=2 * 64 * 128 * pairs / dt / 1e12, unit="TFLOP/s", gpairs_per_s=pairs / dt / 1e9,
                kind="oracle", seconds=dt, **_cpu_fields(oracle),
                sample=f"{len(rows)} query rows of the 64K ADIndex call (evenly spread, the last 16, rows "
                       f"8176..8207 around the first bank group) and the banks of their {len(groups)} groups "
                       f"({pairs} scored pairs), fp64 C oracle with OpenMP",
                parity_of_sampled_gpu_rows=parity)


# ---------------------------------------------------- DSA-shaped bf16 prefill

def bench_dsa16k(dsa, args, log):
    """One layer of DSA-shaped bf16 prefill: T=16384, H=64, d=128, top-2048, one
    call (134,225,920 pairs, 2.199 TFLOP), against the bf16 MFMA peak."""
    from workloads import make_workload
    T, H, d, K = 16384, 64, 128, 2048
    log("generating DSA bf16 prefill inputs T=16384 on the GPU")
    wl = make_workload(2, seed=args.seed, device="cuda")
    t = wl.tensors
    out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.workspace_prefill(T, T, H, d, K, dsa.DSAIDX_BF16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        dsa.indexer_prefill(t["q"], t["k"], t["w"], 0, K, want_score=False, out_idx=out, ws=ws)
    log("timing the 16K bf16 prefill")
    ms, ev = _timed_calls(step, args.steps * 2, stream)
    pairs = _pairs_causal(0, T)
    flops = 2 * H * d * pairs
    tf = flops / (ms * 1e-3) / 1e12
    achieved = flops / (ev * 1e-3) / 1e12
    res = dict(workload="DSA prefill, one layer: T=16384, H=64, d=128, top-2048, bf16", ms_per_call=ms,
               tflops=tf, gpairs_per_s=pairs / (ms * 1e-3) / 1e9, frac_of_bf16_peak=tf / PEAK_BF16_TFLOPS,
               roofline=dict(bound="mfma", kernel="dense_topk_kernel<bf16> (one call: rows of at most "
                                                  "2K + 2048 keys keep their row, the rest stream)",
                             achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                             frac=achieved / PEAK_BF16_TFLOPS, avg_launch_ms=ev, flops_per_launch=flops,
                             traffic=None))
    if not args.no_cpu:
        import oracle
        from tests.parity import compare, pair_refs
        rows = _stratified(T, args.cpu_dsa16k_rows)
        log(f"cpu oracle on {len(rows)} sampled 16K rows")
        h = {k2: v.cpu() for k2, v in t.items()}
        t0 = time.perf_counter()
        ri, rs = oracle.prefill(h["q"], h["k"], h["w"], "bf16", 0, K, rows=rows)
        dt = time.perf_counter() - t0
        spairs = int((rows + 1).sum())
        gi = out[torch.as_tensor(rows, device="cuda")].cpu().numpy()

        score_of, cond_of = pair_refs(h["q"], h["k"], h["w"], rows, "bf16", "bf16")
        parity = _parity("dsa16k", lambda: compare(gi, None, ri, rs, False, score_of, ref_cond_of=cond_of))
        res["cpu_baseline"] = dict(value=2 * H * d * spairs / dt / 1e12, unit="TFLOP/s",
                                   gpairs_per_s=spairs / dt / 1e9, kind="oracle", seconds=dt,
                                   **_cpu_fields(oracle),
                                   sample=f"{len(rows)} query rows of the 16K prefill (evenly spread and the "
                                          f"last 16; {spairs} scored pairs), fp64 C oracle with OpenMP",
                                   parity_of_sampled_gpu_rows=parity)
    return res


# ------------------------------------------------------ layer-wise reuse

TABLE9_DEEPSEEK_MAX = (  # (G, P, layers) of Appendix C.4 Table 9 (DeepSeek-V3.2, max statistic)
    (16, 8192, "2,3,5-8,10,12-14,18,22,37,44"),
    (8, 8192, "0,1,9,15,23,25,34,36,41,42,47,53,54,58,60"),
    (16, 16384, "4,11,16,19,20,24,26-32,35,38-40,48,50-52,56,57,59"),
    (8, 16384, "17,21,33,43,45,46,49,55"),
)


def _layer_list(spec):
    out = []
    for part in spec.split(","):
        a, _, b = part.partition("-")
        out.extend(range(int(a), int(b or a) + 1))
    return out


def bench_layerwise(dsa, args, log, dense_ms=None):
    """The 61 indexer layers of DeepSeek-V3.2 at T=65536, each with the (G, P)
    that Table 9 assigns it, in one indexer_layers call (bf16, H=Hs=64,
    d=128, top-2048; every layer on the same synthetic inputs).  Reported
    against 61 dense layers (the dense 64K layer's time times 61) and against
    Eq. (27)'s scoring-count prediction for prefill."""
    from workloads import make_workload
    T, H, d, K = 65536, 64, 128, 2048
    setting = {}
    for G, P, spec in TABLE9_DEEPSEEK_MAX:
        for layer in _layer_list(spec):
            setting[layer] = (G, P)
    n = len(setting)
    assert sorted(setting) == list(range(61)), "Table 9 covers layers 0..60 once"
    log("generating layer-wise inputs T=65536 bf16 on the GPU")
    wl = make_workload(5, seed=args.seed, device="cuda", T=T)
    t = wl.tensors
    g8w = make_workload(5, seed=args.seed + 1, device="cuda", T=T, G=8)  # a group query for groups of 8
    g8 = dict(qbar=g8w["qbar"], wbar=g8w["wbar"])
    del g8w
    out = torch.empty((T, K), dtype=torch.int32, device="cuda")  # every layer writes here (timing only)
    layers = []
    for layer in range(n):
        G, P = setting[layer]
        src = t if G == 16 else g8
        layers.append(dict(q=t["q"], k=t["k"], w=t["w"], qbar=src["qbar"], wbar=src["wbar"], G=G, P=P,
                           out_idx=out))
    ws = torch.empty(dsa.workspace_layers(layers, T, T, H, d, K, dsa.DSAIDX_BF16), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    log(f"timing {n} layers with Table 9's settings")
    ms, ev = _timed_calls(lambda: dsa.indexer_layers(layers, 0, K, ws=ws), max(1, args.layer_steps), stream)
    Gs = [setting[i][0] for i in range(n)]
    Ps = [setting[i][1] for i in range(n)]
    predicted = dsa.layerwise_speedup(list(zip(Gs, Ps)), T, R=0)
    pairs = sum(dsa.indexer_group_bank_pairs(T, 0, G, P) for G, P in zip(Gs, Ps))
    res = dict(workload=f"layer-wise reuse: DeepSeek-V3.2's 61 indexer layers at T={T}, (G, P) per layer from "
                        "Table 9 (max statistic: 14 x (16, 8K), 15 x (8, 8K), 24 x (16, 16K), 8 x (8, 16K)), "
                        "bf16, H=Hs=64, d=128, top-2048, one indexer_layers call",
               ms_per_call=ms, ms_per_layer=ms / n, pairs=pairs,
               tflops=2 * H * d * pairs / (ms * 1e-3) / 1e12,
               eq27_predicted_speedup=predicted)
    if dense_ms:
        res["dense_ms_61_layers"] = dense_ms * n
        res["measured_speedup_vs_dense"] = dense_ms * n / ms
        res["measured_over_predicted"] = res["measured_speedup_vs_dense"] / predicted
    return res


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


# ------------------------------------------------------------------ profiles

def _short_kernel_name(name):
    """A kernel's name without its return type, namespaces and parameter list
    (the template arguments stay)."""
    for p in ("void ", "dsaidx::", "(anonymous namespace)::"):
        name = name.replace(p, "")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i][:70]
    return name[:70]


def summarize_trace(path):
    """A table of rocprofv3's kernel statistics (kernel_stats.csv), or of a
    kernel trace (kernel_trace.csv) by kernel and grid size."""
    import csv
    rows = list(csv.DictReader(open(path)))
    if rows and "Grid_Size_X" in rows[0]:
        groups = {}
        for r in rows:
            key = (_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
            groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print(f"{'kernel':70s} {'workgroups':>10s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
        for (name, wgs), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            print(f"{name:70s} {wgs:10d} {len(v):6d} {sum(v) / len(v):10.2f} {min(v):10.2f} {max(v):10.2f}")
        return
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print(f"{'kernel':70s} {'calls':>6s} {'total_us':>11s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
    for r in rows:
        name = _short_kernel_name(r["Name"])
        print(f"{name:70s} {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e3:11.1f} "
              f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
              f"{float(r['Percentage']):6.2f}")


# kernels of one measured launch in the traffic records, and the calls one
# `bench.py --steps 1 --warmup 0` makes: 32 prefill chunk calls, 3 + 20 decode
# calls
TRAFFIC_KERNELS = {
    "dense_topk_fp8_prefill128k": (("dense_topk_kernel<2, false, ",), 32),
    "decode_call_decode256k": (("fill_i32_kernel", "decode_scan_kernel<2, 128, 1>", "decode_classify_kernel",
                                "decode_select_kernel", "decode_emit_kernel"), 23),
}


def _counter_sums(path, counter):
    """counter value summed per kernel name, and dispatches per kernel name."""
    import csv
    tot, disp = {}, {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        tot[name] = tot.get(name, 0.0) + float(r["Counter_Value"])
        disp[name] = disp.get(name, 0) + 1
    return tot, disp


def summarize_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes):
    """Write profiles/traffic.json: HBM bytes per measured launch from the
    FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch), each scaled by the
    factor that makes the 5-copy probe read and write its known bytes."""
    cf, _ = _counter_sums(copy_fetch_csv, "FETCH_SIZE")
    cw, _ = _counter_sums(copy_write_csv, "WRITE_SIZE")
    # the five copies only (the probe's source is filled by another kernel first)
    copy_fetch_kib = sum(v for k, v in cf.items() if "copyBuffer" in k) / 5
    copy_write_kib = sum(v for k, v in cw.items() if "copyBuffer" in k) / 5
    ff = copy_bytes / 1024 / copy_fetch_kib
    wf = copy_bytes / 1024 / copy_write_kib
    fetch, fd = _counter_sums(fetch_csv, "FETCH_SIZE")
    write, _ = _counter_sums(write_csv, "WRITE_SIZE")
    out = {"_note": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each "
                    "scaled by the factor that makes a plain device copy of copy_bytes read and write "
                    "copy_bytes; source_sha1 hashes the device sources listed (bench.py ignores a record "
                    "whose hash differs from the sources it runs).",
           "calibration": {"copy_bytes": copy_bytes, "copy_fetch_kib": copy_fetch_kib,
                           "copy_write_kib": copy_write_kib, "fetch_factor": ff, "write_factor": wf}}
    for key, (prefixes, calls) in TRAFFIC_KERNELS.items():
        names = [n for n in fetch if any(n.startswith(p) or ("::" + p) in n or (" " + p) in n for p in prefixes)]
        f_kib = sum(fetch[n] for n in names) / calls
        w_kib = sum(write.get(n, 0.0) for n in names) / calls
        out[key] = {"kernels": sorted(names), "dispatches": [fd[n] for n in sorted(names)], "calls": calls,
                    "fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
                    "hbm_bytes_per_launch": (f_kib * ff + w_kib * wf) * 1024,
                    "source_sha1": _source_sha1(KERNEL_SOURCES[key]), "sources": list(KERNEL_SOURCES[key])}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--cpu-decode-rows", type=int, default=32)
    ap.add_argument("--cpu-dsa16k-rows", type=int, default=1024)
    ap.add_argument("--cpu-adindex-rows", type=int, default=512)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-adindex", action="store_true", help="skip the ADIndex group-bank workload")
    ap.add_argument("--adindex-len", type=int, default=65536, metavar="T",
                    help="sequence length of the ADIndex workload (65536; the pages quote 262144)")
    ap.add_argument("--no-dsa16k", action="store_true", help="skip the 16K bf16 DSA prefill layer")
    ap.add_argument("--no-layerwise", action="store_true", help="skip the 61-layer Table 9 pass")
    ap.add_argument("--layer-steps", type=int, default=1, help="timed 61-layer passes (about 0.7 s each)")
    ap.add_argument("--mtp", action="store_true", help="also time MTP verification windows at 256K")
    ap.add_argument("--calib", action="store_true", help="also time the calibration statistics kernels")
    ap.add_argument("--group-query", action="store_true", help="also time the group query construction")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES device-to-device 5 times (calibrates HBM byte counters)")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="only print a table of a rocprofv3 kernel_stats.csv (no GPU)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="only update profiles/traffic.json from four rocprofv3 counter_collection.csv files "
                         "(FETCH_SIZE and WRITE_SIZE of `bench.py --steps 1 --warmup 0 --no-cpu --no-dsa16k "
                         "--no-adindex --no-layerwise`, then of `bench.py --copy-probe BYTES`; no GPU)")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30, help="the copy probe's BYTES (--summarize-traffic)")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, copy_bytes=args.copy_bytes)
        return

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
        "mfma_ceiling": pre["mfma_ceiling"],
        "cpu_baseline": cpu,
    }
    if not args.no_decode:
        line["decode"] = bench_decode(dsa, args, log)
    if not args.no_dsa16k:
        line["dsa16k"] = bench_dsa16k(dsa, args, log)
        line["dsa16k"]["roofline"]["frac_of_bf16_ceiling"] = (
            line["dsa16k"]["roofline"]["achieved"] / pre["mfma_ceiling"]["bf16"]["tflops"])
    dense64k_ms = None
    if not args.no_adindex:
        line["adindex"] = bench_adindex(dsa, args, log)
        line["adindex"]["roofline"]["frac_of_bf16_ceiling"] = (
            line["adindex"]["roofline"]["achieved"] / pre["mfma_ceiling"]["bf16"]["tflops"])
        dense64k_ms = line["adindex"].pop("_dense_ms")
    if not args.no_layerwise:
        line["layerwise"] = bench_layerwise(dsa, args, log,
                                            dense64k_ms if args.adindex_len == 65536 else None)
    if args.mtp:
        line["mtp"] = bench_mtp(dsa, args, log)
    if args.calib:
        line["calib"] = bench_calib(dsa, args, log)
    if args.group_query:
        line["group_query"] = bench_group_query(dsa, args, log)
    failed = {k: v for k, v in PARITY.items() if v != "ok"}
    if failed:  # a wrong result makes every rate above meaningless
        line["value"] = None
        line["invalid"] = "parity of sampled GPU rows against the oracle failed: " + "; ".join(
            f"{k}: {v}" for k, v in failed.items())
    line["parity"] = dict(PARITY)
    print(json.dumps(line), flush=True)
    if failed:
        sys.exit(1)


if __name__ == "__main__":
    main()
