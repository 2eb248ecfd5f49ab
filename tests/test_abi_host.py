"""The C ABI of libdsaidx.so without a GPU: the library loads, exports every
function the header declares, rejects bad arguments on the host before any
launch (the pointers below are never dereferenced), sizes workspaces, and
plans the group-bank pair count exactly as the oracle counts it."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_indexer.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
BF16, FP8 = 1, 2


@pytest.fixture(scope="module")
def L():
    from sparse_attention_indexer_dsa_amd import _lib
    return _lib.lib()


def P(v):
    """A fake device pointer: aligned, non-null, never dereferenced by validation."""
    return ctypes.c_void_p(v)


A = P(1 << 20)  # 16-byte aligned


def test_header_symbols_exported(L):
    names = re.findall(r"^\s*(?:[\w\s\*]+?)\b(indexer_\w+)\s*\(", open(HEADER).read(), re.M)
    names = sorted(set(names))
    assert len(names) == 25, names
    for n in names:
        assert hasattr(L, n), n


def _prefill(L, **kw):
    a = dict(q=A, qs=None, k=A, ks=None, w=A, dtype=BF16, Tq=16, Tk=16, H=64, d=128, q_pos0=0, topk=8,
             out=A, sc=None, ws=A, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return L.indexer_prefill(a["q"], a["qs"], a["k"], a["ks"], a["w"], a["dtype"], a["Tq"], a["Tk"], a["H"],
                             a["d"], a["q_pos0"], a["topk"], a["out"], a["sc"], a["ws"], a["ws_bytes"],
                             a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(w=None), INVALID),
    (dict(topk=0), INVALID), (dict(topk=4096), UNSUPPORTED), (dict(H=0), INVALID), (dict(H=65), UNSUPPORTED),
    (dict(d=48), UNSUPPORTED), (dict(d=32, dtype=FP8, qs=A, ks=A), UNSUPPORTED), (dict(dtype=3), INVALID),
    (dict(q_pos0=1), INVALID), (dict(Tk=15), INVALID), (dict(Tq=-1), INVALID),
    (dict(q=P((1 << 20) + 4)), INVALID), (dict(out=P((1 << 20) + 8)), INVALID),
    (dict(dtype=FP8), INVALID), (dict(qs=A), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE), (dict(ws=P((1 << 20) + 2)), INVALID),
    (dict(Tk=1 << 31, Tq=1), UNSUPPORTED),
])
def test_prefill_rejects(L, kw, code):
    assert _prefill(L, **kw) == code
    assert len(L.indexer_last_error()) > 0


def test_empty_prefill_is_a_noop(L):
    assert _prefill(L, Tq=0, ws=None, ws_bytes=0) == OK
    assert L.indexer_prefill_workspace_size(0, 16, 64, 128, 8, BF16) == 0


def test_workspace_sizes(L):
    a = L.indexer_prefill_workspace_size(4096, 131072, 64, 128, 2048, FP8)
    b = L.indexer_prefill_workspace_size(8192, 131072, 64, 128, 2048, FP8)
    c = L.indexer_prefill_workspace_size(40000, 131072, 64, 128, 2048, FP8)
    assert 0 < a < b <= c  # capped by the rows of one launch
    assert L.indexer_decode_workspace_size(32, 262144, 64, 128, 2048) >= 32 * 262144 * 4
    g = L.indexer_group_bank_workspace_size(65536, 65536, 64, 64, 128, 16, 8192, 2048, BF16, 0)
    assert g > 0
    # mean pooling adds the pooled bf16 queries and fp32 gates of every complete group
    gp = L.indexer_group_bank_workspace_size(65536, 65536, 64, 64, 128, 16, 8192, 2048, BF16, 2)
    assert gp - g == 4096 * 64 * 128 * 2 + 4096 * 64 * 4


def _decode(L, **kw):
    a = dict(q=A, kc=A, ks=A, w=A, lens=A, B=4, N=1024, H=64, d=128, topk=64, out=A, sc=None, ws=A,
             ws_bytes=1 << 40)
    a.update(kw)
    return L.indexer_decode(a["q"], a["kc"], a["ks"], a["w"], a["lens"], a["B"], a["N"], a["H"], a["d"],
                            a["topk"], a["out"], a["sc"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kc=None), INVALID), (dict(lens=None), INVALID), (dict(B=-1), INVALID), (dict(N=-2), INVALID),
    (dict(d=32), UNSUPPORTED), (dict(topk=5000), UNSUPPORTED), (dict(ks=P((1 << 20) + 2)), INVALID),
    (dict(ws_bytes=10), WORKSPACE), (dict(H=100), UNSUPPORTED),
])
def test_decode_rejects(L, kw, code):
    assert _decode(L, **kw) == code


def _group(L, **kw):
    a = dict(q=A, qs=None, k=A, ks=None, w=A, dtype=BF16, Tq=64, Tk=64, H=8, d=64, q_pos0=0, qbar=A,
             qbs=None, wbar=A, Hs=8, G=16, P=32, topk=8, flags=0, out=A, bank=None, sc=None, ws=A,
             ws_bytes=1 << 40)
    a.update(kw)
    return L.indexer_group_bank(a["q"], a["qs"], a["k"], a["ks"], a["w"], a["dtype"], a["Tq"], a["Tk"], a["H"],
                                a["d"], a["q_pos0"], a["qbar"], a["qbs"], a["wbar"], a["Hs"], a["G"], a["P"],
                                a["topk"], a["flags"], a["out"], a["bank"], a["sc"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(G=5), UNSUPPORTED), (dict(G=32), UNSUPPORTED), (dict(P=4), INVALID), (dict(P=20000), UNSUPPORTED),
    (dict(q_pos0=8, Tk=128), INVALID), (dict(flags=4), INVALID), (dict(qbar=None), INVALID),
    (dict(flags=2), INVALID), (dict(flags=2, qbar=None), INVALID),
    (dict(flags=2, qbar=None, wbar=None, Hs=4), INVALID),
    (dict(flags=2, qbar=None, wbar=None, dtype=FP8, qs=A, ks=A), UNSUPPORTED),
    (dict(Hs=0), INVALID), (dict(Hs=80), UNSUPPORTED), (dict(dtype=FP8, qs=A, ks=A), INVALID),
    (dict(qbs=A), INVALID), (dict(bank=P((1 << 20) + 4)), INVALID), (dict(ws_bytes=1), WORKSPACE),
])
def test_group_bank_rejects(L, kw, code):
    assert _group(L, **kw) == code


@pytest.mark.parametrize("Tq,q_pos0,G,P,flags", [
    (65536, 0, 16, 8192, 0), (131072, 0, 8, 4096, 0), (203, 0, 4, 48, 0), (646, 52, 4, 96, 0),
    (646, 52, 4, 96, 1), (100, 0, 16, 16384, 0), (0, 0, 4, 64, 0),
])
def test_pair_plan_matches_oracle(L, Tq, q_pos0, G, P, flags):
    """The library's launch plan scores exactly the pairs the oracle scores."""
    assert L.indexer_group_bank_pairs(Tq, q_pos0, G, P, flags) == oracle.group_bank_pairs(Tq, q_pos0, G, P, flags)


def test_binding_refuses_host_tensors():
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    q = torch.zeros((4, 4, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dsa.indexer_prefill(q, torch.zeros((4, 32), dtype=torch.bfloat16), torch.zeros((4, 4)), 0, 2)


def _mtp(L, **kw):
    a = dict(q=A, kc=A, ks=A, w=A, qbar=A, wbar=A, lens=A, B=4, N=1024, m=16, H=64, Hs=16, d=128, G=4, P=256,
             topk=64, flags=0, out=A, bank=None, sc=None, ws=A, ws_bytes=1 << 40)
    a.update(kw)
    return L.indexer_mtp(a["q"], a["kc"], a["ks"], a["w"], a["qbar"], a["wbar"], a["lens"], a["B"], a["N"], a["m"],
                         a["H"], a["Hs"], a["d"], a["G"], a["P"], a["topk"], a["flags"], a["out"], a["bank"], a["sc"],
                         a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(G=5), UNSUPPORTED), (dict(m=12, G=8), INVALID), (dict(m=128), UNSUPPORTED), (dict(N=8), INVALID),
    (dict(P=32), INVALID), (dict(P=20000), UNSUPPORTED), (dict(flags=1), INVALID), (dict(flags=2), INVALID),
    (dict(flags=10, qbar=None, wbar=None, Hs=64), INVALID), (dict(flags=16), INVALID),
    (dict(flags=2, qbar=None, wbar=None), INVALID), (dict(qbar=None), INVALID), (dict(lens=None), INVALID),
    (dict(d=32), UNSUPPORTED), (dict(Hs=0), INVALID), (dict(Hs=80), UNSUPPORTED), (dict(B=5000), UNSUPPORTED),
    (dict(ks=P((1 << 20) + 2)), INVALID), (dict(ws_bytes=10), WORKSPACE), (dict(topk=4096), UNSUPPORTED),
])
def test_mtp_rejects(L, kw, code):
    assert _mtp(L, **kw) == code


def test_mtp_pairs_match_oracle(L):
    lens = np.array([1, 100, 2048, 2049, 70000, 131057], np.int32)
    for G in (4, 8, 16):
        got = L.indexer_mtp_pairs(lens.ctypes.data_as(ctypes.c_void_p), len(lens), 131072, 16, G, 2048, 0)
        assert got == oracle.mtp_pairs(lens, 16, G, 2048)
        got = L.indexer_mtp_pairs(lens.ctypes.data_as(ctypes.c_void_p), len(lens), 131072, 16, G, 2048, 8)
        assert got == oracle.mtp_pairs(lens, 16, G, 2048, oracle.NO_BANK)
    # out-of-range prefix lengths count as clamped
    bad = np.array([0, 200000], np.int32)
    got = L.indexer_mtp_pairs(bad.ctypes.data_as(ctypes.c_void_p), 2, 131072, 16, 4, 2048, 0)
    assert got == oracle.mtp_pairs([1, 131057], 16, 4, 2048)



def test_calibration_host_functions_match_oracle(L):
    """The library's scoring-count model, capacity statistics, Eq. (5)
    selection and Eq. (27) aggregation against the oracle's and the printed
    Table 5(c)."""
    import oracle.calib as calib
    import sparse_attention_indexer_dsa_amd as dsa
    golden = os.path.join(ROOT, "tests", "golden", "table5_speedups.txt")
    for line in open(golden):
        if line.startswith("#") or not line.strip() or not line.startswith("c"):
            continue
        _, G, P, *vals = line.split()
        for Lk, v in zip((16384, 32768, 65536, 131072), vals):
            got = dsa.speedup_joint(Lk, int(G), int(P[:-1]) * 1024)
            assert round(got, 2) == float(v), (G, P, Lk, got, v)
    rng = np.random.default_rng(5)
    for _ in range(20):
        stats = {g: float(rng.integers(1000, 40000)) for g in (4, 8, 16)}
        assert dsa.select_setting(stats) == calib.select_setting(stats), stats
        settings = [calib.SETTINGS[i] if i < 9 else None for i in rng.integers(0, 10, size=7)]
        assert abs(dsa.layerwise_speedup(settings, 65536) / calib.layerwise_speedup(settings, 65536) - 1) < 1e-12
    sizes = rng.integers(0, 30000, size=101)
    for st in ("max", "mean", "p90"):
        assert dsa.union_stat(sizes, st) == calib.union_stat(sizes, st)


# ------------------------------------------------------- layer-wise dispatch

def _layers(**per_layer):
    from sparse_attention_indexer_dsa_amd._lib import Layer
    specs = per_layer.get("specs")
    arr = (Layer * len(specs))()
    for i, sp in enumerate(specs):
        arr[i].q, arr[i].k, arr[i].w, arr[i].out_idx = 1 << 20, 1 << 20, 1 << 20, 1 << 20
        for name, v in sp.items():
            setattr(arr[i], name, v)
    return arr


def _call_layers(L, arr, n=None, Tq=64, Tk=64, ws_bytes=1 << 40, topk=8):
    return L.indexer_layers(arr, len(arr) if n is None else n, BF16, Tq, Tk, 64, 128, 0, topk, A, ws_bytes, None)


def test_layers_validate_every_layer_first(L):
    """indexer_layers checks every layer before it enqueues anything, and an
    error names the layer: a bad setting in the last layer fails the call."""
    good_bank = dict(qbar=1 << 20, wbar=1 << 20, Hs=64, G=16, P=16)
    assert _call_layers(L, _layers(specs=[dict(), good_bank]), Tq=0) == OK
    arr = _layers(specs=[dict(), good_bank, dict(good_bank, G=5)])
    assert _call_layers(L, arr) == UNSUPPORTED
    assert "layer 2" in L.indexer_last_error().decode()
    arr = _layers(specs=[dict(qbar=1 << 20)])  # an original-indexer layer takes no group query
    assert _call_layers(L, arr) == INVALID and "layer 0" in L.indexer_last_error().decode()
    arr = _layers(specs=[dict(), dict(good_bank, P=4)])  # P below topk
    assert _call_layers(L, arr) == INVALID and "layer 1" in L.indexer_last_error().decode()
    assert L.indexer_layers(None, 2, BF16, 64, 64, 64, 128, 0, 8, A, 1 << 40, None) == INVALID
    assert _call_layers(L, _layers(specs=[dict()]), n=-1) == INVALID


def test_layers_workspace_is_the_largest_layers(L):
    """The layer call's workspace is the largest need of its layers: the
    original indexer's and each (G, P)'s group-bank workspace."""
    Tq = Tk = 20000
    specs = [dict(), dict(qbar=1 << 20, wbar=1 << 20, Hs=64, G=16, P=8192),
             dict(qbar=1 << 20, wbar=1 << 20, Hs=64, G=8, P=16384)]
    arr = _layers(specs=specs)
    need = L.indexer_layers_workspace_size(arr, 3, Tq, Tk, 64, 128, 2048, BF16)
    want = max(L.indexer_prefill_workspace_size(Tq, Tk, 64, 128, 2048, BF16),
               L.indexer_group_bank_workspace_size(Tq, Tk, 64, 64, 128, 16, 8192, 2048, BF16, 0),
               L.indexer_group_bank_workspace_size(Tq, Tk, 64, 64, 128, 8, 16384, 2048, BF16, 0))
    assert need == want > 0
    assert _call_layers(L, arr, Tq=Tq, Tk=Tk, ws_bytes=1000, topk=2048) == WORKSPACE
    assert "workspace" in L.indexer_last_error().decode()
    assert L.indexer_layers_workspace_size(arr, 0, Tq, Tk, 64, 128, 2048, BF16) == 0


def test_read_probe_rejects(L):
    assert L.indexer_read_probe(A, 1 << 20, A, 0, None) == INVALID
    assert L.indexer_read_probe(P((1 << 20) + 4), 64, A, 8, None) == INVALID
    assert L.indexer_read_probe(A, -1, A, 8, None) == INVALID
    assert L.indexer_read_probe(A, 64, None, 8, None) == INVALID


def test_mfma_probe_rejects(L):
    M = 0x37373737
    assert L.indexer_mfma_probe(FP8, 0, 1, 256, M, A, A, None) == INVALID
    assert L.indexer_mfma_probe(FP8, 16, 3, 256, M, A, A, None) == INVALID
    assert L.indexer_mfma_probe(FP8, 16, 1, 0, M, A, A, None) == INVALID
    assert L.indexer_mfma_probe(FP8, 16, 1, 65536, M, A, A, None) == INVALID
    assert L.indexer_mfma_probe(FP8, 16, 1, 256, M, None, A, None) == INVALID
    assert L.indexer_mfma_probe(FP8, 16, 1, 256, M, A, P(A.value + 4), None) == INVALID
    assert "clocks" in L.indexer_last_error().decode()
    assert L.indexer_mfma_probe(7, 16, 1, 256, M, A, A, None) == INVALID
    # a mask byte that keeps the low seven bits lets E4M3 NaN (S.1111.111) through
    for bad in (0xFFFFFFFF, 0x7F000000, 0x0000007F, 0xFEFE7FFE):
        assert L.indexer_mfma_probe(FP8, 16, 1, 256, bad, A, A, None) == INVALID
        assert "NaN" in L.indexer_last_error().decode()
    # a mask half that keeps every exponent bit lets bf16 infinities and NaNs through
    for bad in (0xFFFFFFFF, 0x7F800000, 0x00007F80, 0xBFFF7F80):
        assert L.indexer_mfma_probe(BF16, 16, 1, 256, bad, A, A, None) == INVALID
        assert "bf16" in L.indexer_last_error().decode()


def test_decode_noalloc_refuses_beyond_its_scratch(L):
    """The allocation-free decode entry point has a fixed scratch array: sizes
    whose workspace exceeds it are refused on the host, before any launch."""
    cap = L.indexer_decode_noalloc_max_bytes()
    assert cap == 96 << 20
    assert L.indexer_decode_workspace_size(32, 262144, 64, 128, 2048) <= cap
    assert L.indexer_decode_workspace_size(64, 262144, 64, 128, 2048) > cap
    rc = L.indexer_decode_noalloc(A, A, A, A, A, 64, 262144, 64, 128, 2048, A, None, None)
    assert rc == UNSUPPORTED and "scratch" in L.indexer_last_error().decode()
