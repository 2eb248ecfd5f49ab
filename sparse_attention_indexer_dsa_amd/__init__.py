"""MI355X (gfx950) DSA lightning indexer: Python binding of libdsaidx.so.

The functions below only marshal arguments: every step of the indexer runs in
the library's HIP kernels.  torch supplies device memory (inputs, outputs and
the workspace) and the current HIP stream.  There is no CPU fallback: calling
without the built library, or with host tensors, raises.

    idx, score = indexer_prefill(q, k, w, q_pos0, topk, q_scale=None, k_scale=None)
    idx, score = indexer_decode(q, k_cache, k_scale, w, seq_lens, topk)
    idx, score, bank = indexer_group_bank(q, k, w, qbar, wbar, q_pos0, G, P, topk, ...)
    idx, score, bank = indexer_group_bank(q, k, w, None, None, q_pos0, G, P, topk,
                                          flags=POOL_MEAN)   # training-free group query
    idx, score, bank = indexer_mtp(q, k_cache, k_scale, w, qbar, wbar, prefix_lens, G, P, topk)
    outs = indexer_layers([dict(q=q, k=k, w=w, qbar=qb, wbar=wb, G=16, P=8192), dict(q=q, k=k, w=w, G=0)],
                          q_pos0, topk)            # per-layer (G, P); G = 0 is the original indexer

Tensors (contiguous, on the GPU): q [Tq,H,d] bf16 or uint8 E4M3 codes,
k [Tk,d] the same dtype, w [Tq,H] fp32, per-token fp32 scales for E4M3.
"""
from __future__ import annotations

import torch

from ._lib import (DSAIDX_BF16, DSAIDX_FORCE_BANK, DSAIDX_FP8_E4M3, DSAIDX_OK,  # noqa: F401
                   DSAIDX_NO_BANK, DSAIDX_POOL_MEAN, LIB_PATH, Layer, last_error, lib)

__all__ = ["indexer_prefill", "indexer_decode", "indexer_decode_noalloc", "indexer_group_bank", "indexer_group_bank_pairs",
           "indexer_layers", "workspace_layers",
           "workspace_prefill", "workspace_decode", "workspace_group_bank", "indexer_mtp", "indexer_mtp_pairs",
           "workspace_mtp", "indexer_group_query", "union_sizes", "topk_overlap", "union_stat", "speedup_joint", "select_setting",
           "layerwise_speedup", "read_probe", "mfma_probe", "FORCE_BANK", "POOL_MEAN", "NO_BANK", "lib",
           "LIB_PATH"]

FORCE_BANK = DSAIDX_FORCE_BANK
POOL_MEAN = DSAIDX_POOL_MEAN
NO_BANK = DSAIDX_NO_BANK


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("indexer tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("indexer tensors must be contiguous")
        dev = t.device if dev is None else dev
    return dev


def _dtype(q):
    if q.dtype == torch.bfloat16:
        return DSAIDX_BF16
    if q.dtype == torch.uint8:
        return DSAIDX_FP8_E4M3
    raise ValueError(f"q dtype {q.dtype}: expected bfloat16 or uint8 E4M3 codes")


def _check(rc, what):
    if rc != DSAIDX_OK:
        raise RuntimeError(f"{what} failed ({rc}): {last_error()}")


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _ws(nbytes, dev, ws):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def workspace_prefill(Tq, Tk, H, d, topk, dtype):
    return lib().indexer_prefill_workspace_size(Tq, Tk, H, d, topk, dtype)


def workspace_decode(B, Nmax, H, d, topk):
    return lib().indexer_decode_workspace_size(B, Nmax, H, d, topk)


def workspace_group_bank(Tq, Tk, H, Hs, d, G, P, topk, dtype, flags=0):
    return lib().indexer_group_bank_workspace_size(Tq, Tk, H, Hs, d, G, P, topk, dtype, flags)


def indexer_group_bank_pairs(Tq, q_pos0, G, P, flags=0):
    return lib().indexer_group_bank_pairs(Tq, q_pos0, G, P, flags)


def indexer_prefill(q, k, w, q_pos0=0, topk=2048, q_scale=None, k_scale=None, want_score=True,
                    out_idx=None, out_score=None, ws=None):
    """Dense causal indexer (Eq. (1)-(2)); returns (idx int32 [Tq,topk], score fp32 or None)."""
    dev = _dev(q, k, w, q_scale, k_scale, out_idx, out_score, ws)
    Tq, H, d = q.shape
    Tk = k.shape[0]
    dt = _dtype(q)
    if out_idx is None:
        out_idx = torch.empty((Tq, topk), dtype=torch.int32, device=dev)
    if want_score and out_score is None:
        out_score = torch.empty((Tq, topk), dtype=torch.float32, device=dev)
    ws = _ws(workspace_prefill(Tq, Tk, H, d, topk, dt), dev, ws)
    rc = lib().indexer_prefill(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), dt, Tq, Tk, H, d,
                               q_pos0, topk, _ptr(out_idx), _ptr(out_score), _ptr(ws),
                               _nbytes(ws), _stream(dev))
    _check(rc, "indexer_prefill")
    return out_idx, out_score


def indexer_decode(q, k_cache, k_scale, w, seq_lens, topk=2048, want_score=True, out_idx=None,
                   out_score=None, ws=None):
    """Decode indexer over an E4M3 cache; returns (idx int32 [B,topk], score fp32 or None)."""
    dev = _dev(q, k_cache, k_scale, w, seq_lens, out_idx, out_score, ws)
    B, H, d = q.shape
    Nmax = k_cache.shape[1]
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.uint8 or seq_lens.dtype != torch.int32:
        raise ValueError("decode takes bf16 q, uint8 E4M3 k_cache and int32 seq_lens")
    if out_idx is None:
        out_idx = torch.empty((B, topk), dtype=torch.int32, device=dev)
    if want_score and out_score is None:
        out_score = torch.empty((B, topk), dtype=torch.float32, device=dev)
    ws = _ws(workspace_decode(B, Nmax, H, d, topk), dev, ws)
    rc = lib().indexer_decode(_ptr(q), _ptr(k_cache), _ptr(k_scale), _ptr(w), _ptr(seq_lens), B, Nmax, H, d,
                              topk, _ptr(out_idx), _ptr(out_score), _ptr(ws), _nbytes(ws),
                              _stream(dev))
    _check(rc, "indexer_decode")
    return out_idx, out_score


def indexer_decode_noalloc(q, k_cache, k_scale, w, seq_lens, topk, out_idx, out_score=None):
    """indexer_decode without a workspace: the library's fixed device scratch
    array serves instead (for callers that cannot allocate, e.g. under graph
    capture).  The outputs are caller tensors; nothing is allocated here."""
    dev = _dev(q, k_cache, k_scale, w, seq_lens, out_idx, out_score)
    B, H, d = q.shape
    Nmax = k_cache.shape[1]
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.uint8 or seq_lens.dtype != torch.int32:
        raise ValueError("decode takes bf16 q, uint8 E4M3 k_cache and int32 seq_lens")
    rc = lib().indexer_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(k_scale), _ptr(w), _ptr(seq_lens), B, Nmax, H,
                                      d, topk, _ptr(out_idx), _ptr(out_score), _stream(dev))
    _check(rc, "indexer_decode_noalloc")
    return out_idx, out_score


def indexer_group_bank(q, k, w, qbar, wbar, q_pos0, G, P, topk=2048, q_scale=None, k_scale=None,
                       qbar_scale=None, flags=0, want_score=True, want_bank=False, out_idx=None,
                       out_score=None, out_bank=None, ws=None):
    """ADIndex bank sharing (Eq. (8), (13), (14)); returns (idx, score or None, bank or None).

    With ``flags & POOL_MEAN`` pass qbar = wbar = None: the group query is the
    mean of each group's own queries and gates (the training-free variant)."""
    dev = _dev(q, k, w, qbar, wbar, q_scale, k_scale, qbar_scale, out_idx, out_score, out_bank, ws)
    Tq, H, d = q.shape
    Tk = k.shape[0]
    Hs = H if qbar is None else qbar.shape[1]
    dt = _dtype(q)
    NG = -(-Tq // G)
    if out_idx is None:
        out_idx = torch.empty((Tq, topk), dtype=torch.int32, device=dev)
    if want_score and out_score is None:
        out_score = torch.empty((Tq, topk), dtype=torch.float32, device=dev)
    if want_bank and out_bank is None:
        out_bank = torch.empty((NG, P), dtype=torch.int32, device=dev)
    ws = _ws(workspace_group_bank(Tq, Tk, H, Hs, d, G, P, topk, dt, flags), dev, ws)
    rc = lib().indexer_group_bank(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), dt, Tq, Tk, H, d,
                                  q_pos0, _ptr(qbar), _ptr(qbar_scale), _ptr(wbar), Hs, G, P, topk, flags,
                                  _ptr(out_idx), _ptr(out_bank), _ptr(out_score), _ptr(ws),
                                  _nbytes(ws), _stream(dev))
    _check(rc, "indexer_group_bank")
    return out_idx, out_score, out_bank


def _layer_structs(layers):
    arr = (Layer * len(layers))()
    for i, L in enumerate(layers):
        for name in ("q", "q_scale", "k", "k_scale", "w", "qbar", "qbar_scale", "wbar", "out_idx", "out_score",
                     "out_bank"):
            setattr(arr[i], name, _ptr(L.get(name)))
        arr[i].Hs = L.get("Hs", 0)
        arr[i].G = L.get("G", 0)
        arr[i].P = L.get("P", 0)
        arr[i].flags = L.get("flags", 0)
    return arr


def workspace_layers(layers, Tq, Tk, H, d, topk, dtype):
    """Workspace bytes of indexer_layers (layers as in indexer_layers)."""
    return lib().indexer_layers_workspace_size(_layer_structs(layers), len(layers), Tq, Tk, H, d, topk, dtype)


def indexer_layers(layers, q_pos0=0, topk=2048, want_score=False, want_bank=False, ws=None):
    """Layer-wise reuse (Section 4.1 Eq. (5); Appendix C.4): one call over
    several layers of the same shapes, each with its own tensors and (G, P).

    ``layers`` is a list of dicts with q, k, w (q_scale, k_scale for E4M3),
    G and P (G = 0: the original indexer), and for G > 0 qbar, wbar (Hs from
    qbar; qbar_scale for E4M3) or flags=POOL_MEAN, optional out_idx,
    out_score, out_bank.  Outputs are allocated where missing (scores and
    banks only when asked for).  Returns the list of (idx, score or None,
    bank or None) per layer."""
    if not layers:
        return []
    L0 = layers[0]
    dev = _dev(*[L.get(n) for L in layers for n in ("q", "q_scale", "k", "k_scale", "w", "qbar", "qbar_scale",
                                                  "wbar", "out_idx", "out_score", "out_bank")], ws)
    Tq, H, d = L0["q"].shape
    Tk = L0["k"].shape[0]
    dt = _dtype(L0["q"])
    full = []
    for L in layers:
        L = dict(L)
        if L["q"].shape != L0["q"].shape or L["k"].shape != L0["k"].shape or _dtype(L["q"]) != dt:
            raise ValueError("every layer of one call has the same q and k shapes and dtype")
        G = L.get("G", 0)
        if G and L.get("qbar") is not None:
            L.setdefault("Hs", L["qbar"].shape[1])
        elif G:
            L.setdefault("Hs", H)
        if L.get("out_idx") is None:
            L["out_idx"] = torch.empty((Tq, topk), dtype=torch.int32, device=dev)
        if want_score and L.get("out_score") is None:
            L["out_score"] = torch.empty((Tq, topk), dtype=torch.float32, device=dev)
        if G and want_bank and L.get("out_bank") is None:
            L["out_bank"] = torch.empty((-(-Tq // G), L["P"]), dtype=torch.int32, device=dev)
        full.append(L)
    arr = _layer_structs(full)
    ws = _ws(lib().indexer_layers_workspace_size(arr, len(full), Tq, Tk, H, d, topk, dt), dev, ws)
    rc = lib().indexer_layers(arr, len(full), dt, Tq, Tk, H, d, q_pos0, topk, _ptr(ws),
                              _nbytes(ws), _stream(dev))
    _check(rc, "indexer_layers")
    return [(L["out_idx"], L.get("out_score"), L.get("out_bank")) for L in full]


def workspace_mtp(B, Nmax, m, H, Hs, d, G, P, topk, flags=0):
    return lib().indexer_mtp_workspace_size(B, Nmax, m, H, Hs, d, G, P, topk, flags)


def indexer_mtp_pairs(prefix_lens, Nmax, m, G, P, flags=0):
    """Scores the MTP call evaluates for these prefix lengths (host ints)."""
    import ctypes
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(prefix_lens, dtype=np.int32))
    return lib().indexer_mtp_pairs(lens.ctypes.data_as(ctypes.c_void_p), len(lens), Nmax, m, G, P, flags)


def indexer_mtp(q, k_cache, k_scale, w, qbar, wbar, prefix_lens, G, P, topk=2048, flags=0, want_score=True,
                want_bank=False, out_idx=None, out_score=None, out_bank=None, ws=None):
    """MTP target verification with bank sharing (Section 4.3; Appendix A.2).

    q [B,m,H,d] bf16, k_cache [B,Nmax,d] uint8 E4M3, k_scale [B,Nmax] fp32,
    w [B,m,H], qbar [B,m/G,Hs,d] bf16 and wbar [B,m/G,Hs] (None with
    POOL_MEAN; not read with NO_BANK), prefix_lens [B] int32 on the GPU.  Returns (idx [B,m,topk],
    score or None, bank [B,m/G,P] or None)."""
    dev = _dev(q, k_cache, k_scale, w, qbar, wbar, prefix_lens, out_idx, out_score, out_bank, ws)
    B, m, H, d = q.shape
    Nmax = k_cache.shape[1]
    Hs = H if qbar is None else qbar.shape[2]
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.uint8 or prefix_lens.dtype != torch.int32:
        raise ValueError("MTP takes bf16 q, uint8 E4M3 k_cache and int32 prefix_lens")
    if out_idx is None:
        out_idx = torch.empty((B, m, topk), dtype=torch.int32, device=dev)
    if want_score and out_score is None:
        out_score = torch.empty((B, m, topk), dtype=torch.float32, device=dev)
    if want_bank and out_bank is None:
        out_bank = torch.empty((B, m // G, P), dtype=torch.int32, device=dev)
    ws = _ws(workspace_mtp(B, Nmax, m, H, Hs, d, G, P, topk, flags), dev, ws)
    rc = lib().indexer_mtp(_ptr(q), _ptr(k_cache), _ptr(k_scale), _ptr(w), _ptr(qbar), _ptr(wbar), _ptr(prefix_lens),
                           B, Nmax, m, H, Hs, d, G, P, topk, flags, _ptr(out_idx), _ptr(out_bank), _ptr(out_score),
                           _ptr(ws), _nbytes(ws), _stream(dev))
    _check(rc, "indexer_mtp")
    return out_idx, out_score, out_bank


# ------------------------------------------------------------ calibration

def union_sizes(topk_idx, G, out=None):
    """Eq. (4): union size of the index sets of each complete group of G rows
    of topk_idx [T, K] int32 (GPU); returns int32 [T // G] on the GPU."""
    dev = _dev(topk_idx, out)
    T, K = topk_idx.shape
    if topk_idx.dtype != torch.int32:
        raise ValueError("topk_idx must be int32")
    if out is None:
        out = torch.empty((T // G,), dtype=torch.int32, device=dev)
    _check(lib().indexer_union_sizes(_ptr(topk_idx), T, K, G, _ptr(out), _stream(dev)), "indexer_union_sizes")
    return out


def topk_overlap(a, b, out=None):
    """|A_i ∩ B_i| per row of two int32 [n, K] index-set arrays (GPU)."""
    dev = _dev(a, b, out)
    n, K = a.shape
    if a.shape != b.shape or a.dtype != torch.int32 or b.dtype != torch.int32:
        raise ValueError("a and b must be int32 of the same shape")
    if out is None:
        out = torch.empty((n,), dtype=torch.int32, device=dev)
    _check(lib().indexer_topk_overlap(_ptr(a), _ptr(b), n, K, _ptr(out), _stream(dev)), "indexer_topk_overlap")
    return out


def union_stat(sizes, stat="max"):
    """Capacity statistic of union sizes (host ints): 'max', 'mean' or 'p90'."""
    import ctypes
    import numpy as np
    v = np.ascontiguousarray(np.asarray(sizes, dtype=np.int32))
    r = lib().indexer_union_stat(v.ctypes.data_as(ctypes.c_void_p), len(v), {"max": 0, "mean": 1, "p90": 2}[stat])
    if r < 0:
        raise ValueError("indexer_union_stat: bad arguments")
    return r


def speedup_joint(L, G, P, R=32, m=16, a=8):
    return lib().indexer_speedup_joint(float(L), G, P, R, m, float(a))


def select_setting(stat_by_G, L=131072, R=32, m=16, a=8):
    """Eq. (5): the feasible (G, P) with the largest joint speedup, or None."""
    import ctypes
    st = (ctypes.c_double * 3)(*[float(stat_by_G[g]) for g in (4, 8, 16)])
    G, P = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().indexer_select_setting(st, float(L), R, m, float(a), ctypes.byref(G), ctypes.byref(P)),
           "indexer_select_setting")
    return None if G.value == 0 else (G.value, P.value)


def layerwise_speedup(settings, L, R=32, m=16, a=8):
    """Eq. (27), joint: settings is a list of (G, P) or None per layer."""
    import ctypes
    n = len(settings)
    Gs = (ctypes.c_int * n)(*[0 if s is None else s[0] for s in settings])
    Ps = (ctypes.c_int * n)(*[0 if s is None else s[1] for s in settings])
    r = lib().indexer_layerwise_speedup(Gs, Ps, n, float(L), R, m, float(a))
    if r < 0:
        raise ValueError("indexer_layerwise_speedup: bad arguments")
    return r


def read_probe(buf, nblocks=2048, out=None):
    """Read every byte of the GPU tensor ``buf`` once (the plain read stream
    the memory-bound kernels are measured against); returns the per-workgroup
    XOR words (int32 [nblocks], GPU)."""
    dev = _dev(buf, out)
    if out is None:
        out = torch.empty((nblocks,), dtype=torch.int32, device=dev)
    nbytes = buf.numel() * buf.element_size()
    _check(lib().indexer_read_probe(_ptr(buf), nbytes, _ptr(out), nblocks, _stream(dev)), "indexer_read_probe")
    return out


def mfma_probe(iters, waves_per_simd, nblocks, operand_mask=0x37373737, out=None, clocks=None, device="cuda",
               dtype="fp8"):
    """Run the matrix-core stream (nblocks workgroups of waves_per_simd waves
    per SIMD, each wave 4 * iters 32x32x64 E4M3 MFMAs, or 32x32x16 bf16 MFMAs
    for dtype "bf16", on operand words under operand_mask); returns (out,
    clocks): the lanes' accumulator sums (float32, GPU) and each wave's
    shader-clock and 100 MHz constant-clock counts around its loop (int64
    [waves, 2], GPU)."""
    waves = nblocks * 4 * waves_per_simd
    if out is None:
        out = torch.empty((nblocks * 256 * waves_per_simd,), dtype=torch.float32, device=device)
    if clocks is None:
        clocks = torch.empty((waves, 2), dtype=torch.int64, device=out.device)
    dev = _dev(out, clocks)
    dt = {"fp8": DSAIDX_FP8_E4M3, "bf16": DSAIDX_BF16}[dtype]
    _check(lib().indexer_mfma_probe(dt, int(iters), int(waves_per_simd), int(nblocks), int(operand_mask),
                                    _ptr(out), _ptr(clocks), _stream(dev)), "indexer_mfma_probe")
    return out, clocks


# ------------------------------------------------- group query (Eq. (6)-(7))

def indexer_group_query(c, h, w_pool, w_q, w_g, G, Hs, d, q_pos0=0, rope_dim=64, rope_base=10000.0,
                        qbar=None, wbar=None, ws=None):
    """The group indexer's query and gates from the query latents c [Tq, dc]
    and hidden states h [Tq, dh] (bf16, GPU): returns (qbar bf16
    [ceil(Tq/G), Hs, d], wbar fp32 [ceil(Tq/G), Hs])."""
    dev = _dev(c, h, w_pool, w_q, w_g, qbar, wbar, ws)
    Tq, dc = c.shape
    dh = h.shape[1]
    for t in (c, h, w_pool, w_q, w_g):
        if t.dtype != torch.bfloat16:
            raise ValueError("group query inputs and weights are bf16")
    NG = -(-Tq // G)
    if qbar is None:
        qbar = torch.empty((NG, Hs, d), dtype=torch.bfloat16, device=dev)
    if wbar is None:
        wbar = torch.empty((NG, Hs), dtype=torch.float32, device=dev)
    ws = _ws(lib().indexer_group_query_workspace_size(Tq, dc, dh, Hs, d, G), dev, ws)
    rc = lib().indexer_group_query(_ptr(c), _ptr(h), _ptr(w_pool), _ptr(w_q), _ptr(w_g), Tq, dc, dh, Hs, d, G, q_pos0,
                                   rope_dim, float(rope_base), _ptr(qbar), _ptr(wbar), _ptr(ws),
                                   _nbytes(ws), _stream(dev))
    _check(rc, "indexer_group_query")
    return qbar, wbar
