"""CPU oracle for the DSA lightning indexer and the ADIndex group token bank.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of
the benchmark use it; the GPU library never does.  The arithmetic lives in
``oracle.c`` (plain C, fp64); this module compiles it with gcc and marshals
host arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

F32, BF16, E4M3 = 0, 1, 2
FORCE_BANK = 1
WINDOW = 4  # group_bank flag: MTP window, eligibility decided on the first query
NO_BANK = 8  # every group (MTP: every window) uses the original indexer

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP over queries)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        stale = not os.path.exists(LIB_PATH) or any(
            os.path.getmtime(os.path.join(_HERE, f)) > os.path.getmtime(LIB_PATH) for f in ("oracle.c", "oracle.h"))
        if stale:  # built from older sources: rebuild rather than bind a mismatched library
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_e4m3_to_double.restype = D
        L.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_bf16_to_double.restype = D
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_max_threads.restype = I32
        L.oracle_score_pairs.restype = I32
        L.oracle_score_pairs.argtypes = [P, P, I32, P, P, I32, P, I32, I32, P, P, I64, P, I32]
        L.oracle_score_pairs_cond.restype = I32
        L.oracle_score_pairs_cond.argtypes = [P, P, I32, P, P, I32, P, I32, I32, P, P, I64, P, I32]
        L.oracle_prefill.restype = I32
        L.oracle_prefill.argtypes = [P, P, P, P, P, I32, I64, I64, I32, I32, I64, I32, P, I64, P, P, I32]
        L.oracle_decode.restype = I32
        L.oracle_decode.argtypes = [P, P, P, P, P, I32, I64, I32, I32, I32, P, I64, P, P, I32]
        L.oracle_group_bank.restype = I32
        L.oracle_group_bank.argtypes = [P, P, P, P, P, I32, I64, I64, I32, I32, I64, P, P, P, I32, I32,
                                        I32, I32, ctypes.c_uint, P, I64, P, P, P, P, I32]
        L.oracle_pool_mean_bf16.restype = I32
        L.oracle_pool_mean_bf16.argtypes = [P, P, I64, I32, I32, I32, P, P]
        L.oracle_mtp.restype = I32
        L.oracle_mtp.argtypes = [P, P, P, P, P, P, P, I32, I64, I32, I32, I32, I32, I32, I32, I32,
                                 ctypes.c_uint, P, I64, P, P, P, P, I32]
        L.oracle_mtp_pairs.restype = I64
        L.oracle_mtp_pairs.argtypes = [P, I32, I32, I32, I32, ctypes.c_uint]
        L.oracle_group_bank_pairs.restype = I64
        L.oracle_group_bank_pairs.argtypes = [I64, I64, I32, I32, ctypes.c_uint]
        for name in ("oracle_cost_prefill_base",):
            getattr(L, name).restype = D
            getattr(L, name).argtypes = [D]
        L.oracle_cost_prefill_reuse.restype = D
        L.oracle_cost_prefill_reuse.argtypes = [D, D, D]
        L.oracle_cost_mtp_base_round.restype = D
        L.oracle_cost_mtp_base_round.argtypes = [D, I32]
        L.oracle_cost_mtp_reuse_round.restype = D
        L.oracle_cost_mtp_reuse_round.argtypes = [D, I32, D, I32]
        L.oracle_speedup_joint.restype = D
        L.oracle_speedup_joint.argtypes = [D, I32, D, I32, I32, D]
        _lib = L
    return _lib


# ------------------------------------------------------------------ marshalling

def _host(x):
    """A contiguous host numpy array holding exactly the bytes of ``x``."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16)
            x = x.cpu().contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(dtype: str) -> int:
    return {"f32": F32, "bf16": BF16, "fp8": E4M3}[dtype]


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, len(r)


def prefill(q, k, w, dtype, q_pos0, topk, q_scale=None, k_scale=None, rows=None, nthreads=0):
    """Dense indexer (Eq. 1-2) for every query row (or ``rows``).

    Returns (idx int32 [n,topk], score float64 [n,topk]).
    """
    q, k, w = _host(q), _host(k), _host(w).astype(np.float32)
    q_scale, k_scale = _host(q_scale), _host(k_scale)
    Tq, H, d = q.shape
    Tk = k.shape[0]
    r, nr = _rows(rows)
    n = nr if r is not None else Tq
    idx = np.empty((n, topk), np.int32)
    sc = np.empty((n, topk), np.float64)
    rc = lib().oracle_prefill(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), _dtype_code(dtype),
                              Tq, Tk, H, d, q_pos0, topk, _ptr(r), nr, _ptr(idx), _ptr(sc), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_prefill failed ({rc})")
    return idx, sc


def score_pairs(q, k, w, rows, keys, q_dtype, k_dtype, q_scale=None, k_scale=None, nthreads=0):
    """Eq. (1) for the pairs (q row rows[p], k row keys[p]); q [*,H,d], k [*,d]
    (a decode cache may be passed flattened to [B*Nmax, d])."""
    q, k, w = _host(q), _host(k), _host(w).astype(np.float32)
    q_scale, k_scale = _host(q_scale), _host(k_scale)
    H, d = q.shape[-2], q.shape[-1]
    r = np.ascontiguousarray(np.asarray(rows, np.int64).ravel())
    kk = np.ascontiguousarray(np.asarray(keys, np.int64).ravel())
    assert r.shape == kk.shape
    out = np.empty(len(r), np.float64)
    rc = lib().oracle_score_pairs(_ptr(q), _ptr(q_scale), _dtype_code(q_dtype), _ptr(k), _ptr(k_scale),
                                  _dtype_code(k_dtype), _ptr(w), H, d, _ptr(r), _ptr(kk), len(r), _ptr(out),
                                  nthreads)
    if rc != 0:
        raise ValueError(f"oracle_score_pairs failed ({rc})")
    return out


def score_pairs_cond(q, k, w, rows, keys, q_dtype, k_dtype, q_scale=None, k_scale=None, nthreads=0):
    """The absolute condition of Eq. (1) for the same pairs as score_pairs:
    sum_j |w_j| sum_c |q_jc| |k_c| in fp64 from the dequantised inputs."""
    q, k, w = _host(q), _host(k), _host(w).astype(np.float32)
    q_scale, k_scale = _host(q_scale), _host(k_scale)
    H, d = q.shape[-2], q.shape[-1]
    r = np.ascontiguousarray(np.asarray(rows, np.int64).ravel())
    kk = np.ascontiguousarray(np.asarray(keys, np.int64).ravel())
    assert r.shape == kk.shape
    out = np.empty(len(r), np.float64)
    rc = lib().oracle_score_pairs_cond(_ptr(q), _ptr(q_scale), _dtype_code(q_dtype), _ptr(k), _ptr(k_scale),
                                       _dtype_code(k_dtype), _ptr(w), H, d, _ptr(r), _ptr(kk), len(r), _ptr(out),
                                       nthreads)
    if rc != 0:
        raise ValueError(f"oracle_score_pairs_cond failed ({rc})")
    return out


def decode(q, k_cache, k_scale, w, seq_lens, topk, rows=None, nthreads=0):
    """Decode indexer: one bf16 query per sequence against an E4M3 cache."""
    q, k_cache, k_scale = _host(q), _host(k_cache), _host(k_scale)
    w = _host(w).astype(np.float32)
    seq = _host(seq_lens).astype(np.int32)
    B, H, d = q.shape
    Nmax = k_cache.shape[1]
    r, nr = _rows(rows)
    n = nr if r is not None else B
    idx = np.empty((n, topk), np.int32)
    sc = np.empty((n, topk), np.float64)
    rc = lib().oracle_decode(_ptr(q), _ptr(k_cache), _ptr(k_scale), _ptr(w), _ptr(seq), B, Nmax, H, d,
                             topk, _ptr(r), nr, _ptr(idx), _ptr(sc), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_decode failed ({rc})")
    return idx, sc


POOL_MEAN = 2  # group_bank flag: the training-free group query (mean pooling)


def pool_mean_bf16(q, w, G):
    """Mean-pooled group query of the training-free variant (Section 5 Abl. 2;
    Appendix B.3, B.4): (qbar uint16 bf16 bits [ceil(Tq/G), H, d], wbar float32
    [ceil(Tq/G), H]).  q is bf16 (a torch bfloat16 tensor or uint16 bits)."""
    q, w = _host(q), _host(w).astype(np.float32)
    q = np.ascontiguousarray(q.view(np.uint16))
    Tq, H, d = q.shape
    NG = -(-Tq // G)
    qbar = np.empty((NG, H, d), np.uint16)
    wbar = np.empty((NG, H), np.float32)
    rc = lib().oracle_pool_mean_bf16(_ptr(q), _ptr(w), Tq, H, d, G, _ptr(qbar), _ptr(wbar))
    if rc != 0:
        raise ValueError(f"oracle_pool_mean_bf16 failed ({rc})")
    return qbar, wbar


def group_bank(q, k, w, qbar, wbar, dtype, q_pos0, G, P, topk, flags=0, q_scale=None, k_scale=None,
               qbar_scale=None, rows=None, want_bank=False, nthreads=0):
    """ADIndex bank sharing (Eq. 8, 13, 14) with fallback to the original indexer.

    With ``flags & POOL_MEAN`` the group query is the mean-pooled one of the
    training-free variant (qbar and wbar are ignored; bf16 only).
    Returns (idx [n,topk], score [n,topk], bank [NG,P] or None, pairs).
    """
    if flags & POOL_MEAN:
        if dtype != "bf16":
            raise ValueError("mean pooling takes bf16 queries")
        qbar, wbar = pool_mean_bf16(q, w, G)
        flags &= ~POOL_MEAN
    q, k, w = _host(q), _host(k), _host(w).astype(np.float32)
    qbar, wbar = _host(qbar), _host(wbar).astype(np.float32)
    q_scale, k_scale, qbar_scale = _host(q_scale), _host(k_scale), _host(qbar_scale)
    Tq, H, d = q.shape
    Tk = k.shape[0]
    NG, Hs, _ = qbar.shape
    r, nr = _rows(rows)
    n = nr if r is not None else Tq
    idx = np.empty((n, topk), np.int32)
    sc = np.empty((n, topk), np.float64)
    bank = np.empty((NG, P), np.int32) if want_bank else None
    pairs = ctypes.c_int64(0)
    rc = lib().oracle_group_bank(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), _dtype_code(dtype),
                                 Tq, Tk, H, d, q_pos0, _ptr(qbar), _ptr(qbar_scale), _ptr(wbar), Hs, G, P,
                                 topk, flags, _ptr(r), nr, _ptr(idx), _ptr(sc), _ptr(bank),
                                 ctypes.cast(ctypes.pointer(pairs), ctypes.c_void_p), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_group_bank failed ({rc})")
    return idx, sc, bank, pairs.value


def mtp(q, k_cache, k_scale, w, qbar, wbar, prefix_lens, G, P, topk, flags=0, rows=None, want_bank=False,
        nthreads=0):
    """MTP target verification (Section 4.3; Appendix A.2): windows of m bf16
    queries [B,m,H,d] over E4M3 caches [B,Nmax,d]; N_b = prefix_lens[b] keys
    visible to each window's first query.  ``flags & POOL_MEAN`` pools each
    group's own queries and gates (qbar, wbar ignored); ``flags & NO_BANK``
    sends every window to the original indexer.  Rows index [B*m].
    Returns (idx [n,topk], score [n,topk], bank [B,m/G,P] or None, pairs)."""
    q, k_cache, k_scale = _host(q), _host(k_cache), _host(k_scale)
    w = _host(w).astype(np.float32)
    B, m, H, d = q.shape
    Nmax = k_cache.shape[1]
    if flags & POOL_MEAN:
        pooled = [pool_mean_bf16(q[b], w[b], G) for b in range(B)]
        qbar = np.stack([p[0] for p in pooled])
        wbar = np.stack([p[1] for p in pooled])
    else:
        qbar, wbar = _host(qbar), _host(wbar).astype(np.float32)
    qbar = np.ascontiguousarray(np.asarray(qbar).view(np.uint16))
    Hs = qbar.shape[2]
    lens = np.ascontiguousarray(_host(prefix_lens).astype(np.int32))
    r, nr = _rows(None if rows is None else np.unique(rows))
    if rows is not None and len(np.unique(rows)) != len(rows):
        raise ValueError("rows must be distinct")
    order = None if rows is None else np.argsort(np.argsort(np.asarray(rows)))
    n = nr if r is not None else B * m
    idx = np.empty((n, topk), np.int32)
    sc = np.empty((n, topk), np.float64)
    bank = np.empty((B, m // G, P), np.int32) if want_bank else None
    pairs = ctypes.c_int64(0)
    rc = lib().oracle_mtp(_ptr(q), _ptr(k_cache), _ptr(k_scale), _ptr(w), _ptr(qbar), _ptr(wbar), _ptr(lens), B,
                          Nmax, m, H, Hs, d, G, P, topk, flags & NO_BANK, _ptr(r), nr, _ptr(idx), _ptr(sc),
                          _ptr(bank),
                          ctypes.cast(ctypes.pointer(pairs), ctypes.c_void_p), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_mtp failed ({rc})")
    if order is not None:  # back to the caller's row order
        idx, sc = idx[order], sc[order]
    return idx, sc, bank, pairs.value


def mtp_pairs(prefix_lens, m, G, P, flags=0) -> int:
    lens = np.ascontiguousarray(np.asarray(prefix_lens, np.int32))
    return lib().oracle_mtp_pairs(_ptr(lens), len(lens), m, G, P, flags & NO_BANK)


def group_bank_pairs(Tq, q_pos0, G, P, flags=0) -> int:
    return lib().oracle_group_bank_pairs(Tq, q_pos0, G, P, flags)


def e4m3_to_double(code: int) -> float:
    return lib().oracle_e4m3_to_double(code)


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(bits & 0xFFFF)


def cost_prefill_base(L):
    return lib().oracle_cost_prefill_base(L)


def cost_prefill_reuse(L, G, P):
    return lib().oracle_cost_prefill_reuse(L, G, P)


def cost_mtp_base_round(N, m=16):
    return lib().oracle_cost_mtp_base_round(N, m)


def cost_mtp_reuse_round(N, G, P, m=16):
    return lib().oracle_cost_mtp_reuse_round(N, G, P, m)


def speedup_joint(L, G, P, R=32, m=16, a=8):
    return lib().oracle_speedup_joint(L, G, P, R, m, a)


def max_threads() -> int:
    return lib().oracle_max_threads()
