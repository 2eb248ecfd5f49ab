"""GPU parity at sizes the oracle finishes in seconds: several 32-key tiles, ragged
tails, compaction of the candidate buffer, edge cases.  Every call goes through
the C ABI of libdsaidx.so (via the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import compare, pair_refs
from workloads import make_decode, make_group_bank, make_mtp, make_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsa_amd as m
    m.lib()  # raises if the library is not built
    return m


def _np(t):
    return t.cpu().numpy()


def _rows(Tq, n=48, seed=0):
    """Sampled query rows: the first and last few, plus random ones."""
    if Tq <= n:
        return np.arange(Tq)
    rng = np.random.default_rng(seed)
    head = np.arange(min(4, Tq))
    tail = np.arange(Tq - 4, Tq)
    mid = rng.choice(Tq, n - 8, replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


def _prefill_check(dsa, wl, rows=None, exact=None, topk=None, chunk=None):
    p = wl.params
    K = topk or p["topk"]
    dt = wl.dtype
    dev = "cuda"
    t = {k: v.to(dev) for k, v in wl.tensors.items()}
    q_pos0 = p["q_pos0"]
    Tq = p["Tq"]
    if chunk is None:
        gi, gs = dsa.indexer_prefill(t["q"], t["k"], t["w"], q_pos0, K, t.get("q_scale"), t.get("k_scale"))
    else:
        gi = torch.empty((Tq, K), dtype=torch.int32, device=dev)
        gs = torch.empty((Tq, K), dtype=torch.float32, device=dev)
        for c0 in range(0, Tq, chunk):
            c1 = min(Tq, c0 + chunk)
            Tk = q_pos0 + c1
            dsa.indexer_prefill(t["q"][c0:c1], t["k"][:Tk], t["w"][c0:c1], q_pos0 + c0, K,
                                None if "q_scale" not in t else t["q_scale"][c0:c1],
                                None if "k_scale" not in t else t["k_scale"][:Tk],
                                out_idx=gi[c0:c1], out_score=gs[c0:c1])
    torch.cuda.synchronize()
    rows = np.arange(Tq) if rows is None else np.asarray(rows)
    ri, rs = oracle.prefill(wl["q"], wl["k"], wl["w"], dt, q_pos0, K, wl.tensors.get("q_scale"),
                            wl.tensors.get("k_scale"), rows=rows)
    exact = (p["dist"] == "int") if exact is None else exact

    score_of, cond_of = pair_refs(wl["q"], wl["k"], wl["w"], rows, dt, dt, wl.tensors.get("q_scale"),
                                  wl.tensors.get("k_scale"))
    compare(_np(gi)[rows], _np(gs)[rows], ri, rs, exact, score_of, ref_cond_of=cond_of)
    return gi, gs


def test_config1_tiny_exact(dsa):
    """T=1024, H=4, d=32, K=64, integer inputs: every row bit-exact."""
    wl = make_prefill(T=1024, H=4, d=32, topk=64, dtype="bf16", dist="int", seed=0, w_lo=0, w_hi=3)
    _prefill_check(dsa, wl)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_h64_integer_exact(dsa, dtype):
    """64 heads, d=128, signed integer q, k, w: ties everywhere, sums exact."""
    wl = make_prefill(T=1123, H=64, d=128, topk=100, dtype=dtype, dist="int", seed=1)
    _prefill_check(dsa, wl, rows=_rows(1123, 40, 1))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_h64_random_tolerance(dsa, dtype):
    wl = make_prefill(T=1500, H=64, d=128, topk=256, dtype=dtype, dist="normal", seed=2, Tq=700)
    _prefill_check(dsa, wl, rows=_rows(700, 40, 2))


@pytest.mark.parametrize("H,d,K,T", [(1, 32, 1, 5), (5, 64, 7, 333), (33, 32, 64, 97), (64, 64, 2048, 150),
                                     (17, 128, 33, 1), (2, 32, 64, 2)])
def test_shapes_exact(dsa, H, d, K, T):
    wl = make_prefill(T=T, H=H, d=d, topk=K, dtype="bf16", dist="int", seed=H * 7 + d)
    _prefill_check(dsa, wl, rows=_rows(T, 40, 3))


def test_fp8_shapes_exact(dsa):
    wl = make_prefill(T=260, H=20, d=64, topk=50, dtype="fp8", dist="int", seed=4)
    _prefill_check(dsa, wl)


def test_zero_and_negative_weights(dsa):
    """w = -0: all scores are zero and rank by index; negative w makes many -0
    products that must rank as +0."""
    wl = make_prefill(T=400, H=8, d=32, topk=64, dtype="bf16", dist="int", seed=5)
    wl.tensors["w"] = -torch.zeros_like(wl["w"])
    gi, gs = _prefill_check(dsa, wl)
    assert (_np(gi)[399] == np.arange(64)).all()
    wl2 = make_prefill(T=400, H=8, d=32, topk=64, dtype="bf16", dist="int", seed=6, w_lo=-3, w_hi=0)
    _prefill_check(dsa, wl2)


@pytest.mark.parametrize("H,d", [(64, 128), (16, 64)])
def test_zero_key_scales_signed_gates(dsa, H, d):
    """Integer E4M3 inputs where every fifth key token has scale 0 and the
    gates have both signs: a negative head sum times a zero scale is -0, which
    must rank as +0 (ties then go to the lower index), in the dense kernel
    (64 heads, d = 128) and the general one; decode sees the same cache."""
    T, K = 700, 96
    wl = make_prefill(T=T, H=H, d=d, topk=K, dtype="fp8", dist="int", seed=20 + H)
    ks = wl["k_scale"].clone()
    ks[::5] = 0.0
    wl.tensors["k_scale"] = ks
    _prefill_check(dsa, wl, rows=_rows(T, 40, 20 + H))
    B, N = 3, 900
    wd = make_decode(B, N, H, d, K, dist="int", seed=30 + H, seq_lens=[900, 333, 4])
    kd = wd["k_scale"].clone()
    kd[:, ::5] = 0.0
    wd.tensors["k_scale"] = kd
    _decode_check(dsa, wd)


@pytest.mark.parametrize("H,d,dtype", [(64, 128, "bf16"), (64, 128, "fp8"), (24, 64, "bf16")])
def test_all_negative_gates_random(dsa, H, d, dtype):
    """Normal inputs with every gate negative, w = -|N(0,1)|/8: every score is
    at most 0 and the top K are the keys whose heads are least positive.  This
    is where the dense kernel's (w/2)|s| + (w/2)s split of the ReLU sum
    cancels most; the tolerance rule must still hold."""
    T, Tq, K = 3000, 400, 256
    wl = make_prefill(T=T, H=H, d=d, topk=K, dtype=dtype, dist="normal", seed=40 + H, Tq=Tq)
    g = torch.Generator().manual_seed(41 + H)
    wl.tensors["w"] = -(torch.randn((Tq, H), generator=g).abs() / 8)
    gi, gs = _prefill_check(dsa, wl, rows=_rows(Tq, 40, 40 + H))
    v = _np(gs)[_np(gi) >= 0]
    assert (v <= 0).all()


def test_compaction_many_rounds(dsa):
    """Small K over a long prefix: the candidate buffer fills and compacts many
    times; increasing scores (every key beats the threshold) plus ties."""
    T, d, K = 6000, 32, 16
    q = torch.ones((T, 1, d), dtype=torch.float32)
    s = torch.arange(T)
    k = torch.zeros((T, d), dtype=torch.float32)
    k[s, s % d] = (s // 24 + 1).clamp(max=250).float()  # non-decreasing with long tie runs
    wl = make_prefill(T=T, H=1, d=d, topk=K, dtype="bf16", dist="int", seed=7)
    wl.tensors.update(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), w=torch.ones((T, 1)))
    _prefill_check(dsa, wl, rows=_rows(T, 40, 7), exact=True)
    # random integer data, K small: several compactions at realistic rates
    wl2 = make_prefill(T=5000, H=16, d=64, topk=24, dtype="bf16", dist="int", seed=8)
    _prefill_check(dsa, wl2, rows=_rows(5000, 40, 8))


def test_chunked_equals_unchunked(dsa):
    wl = make_prefill(T=2100, H=64, d=128, topk=128, dtype="bf16", dist="normal", seed=9)
    gi, gs = _prefill_check(dsa, wl, rows=_rows(2100, 24, 9))
    ci, cs = _prefill_check(dsa, wl, rows=_rows(2100, 24, 10), chunk=512)
    assert torch.equal(gi, ci) and torch.equal(gs, cs)


def test_deterministic(dsa):
    wl = make_prefill(T=1800, H=64, d=128, topk=512, dtype="fp8", dist="normal", seed=10)
    t = {k: v.cuda() for k, v in wl.tensors.items()}
    a = dsa.indexer_prefill(t["q"], t["k"], t["w"], 0, 512, t["q_scale"], t["k_scale"])
    b = dsa.indexer_prefill(t["q"], t["k"], t["w"], 0, 512, t["q_scale"], t["k_scale"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# --- the dense kernel (33..64 heads, d = 128): head padding, the ReLU identity
# with zero and negative weights, compaction, partial workgroups, K > prefix

@pytest.mark.parametrize("H,dtype", [(33, "bf16"), (40, "fp8"), (63, "bf16"), (48, "fp8")])
def test_dense_kernel_head_counts(dsa, H, dtype):
    wl = make_prefill(T=900, H=H, d=128, topk=96, dtype=dtype, dist="int", seed=H)
    _prefill_check(dsa, wl, rows=_rows(900, 32, H))
    wl2 = make_prefill(T=700, H=H, d=128, topk=64, dtype=dtype, dist="normal", seed=H + 1)
    _prefill_check(dsa, wl2, rows=_rows(700, 32, H + 1))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_dense_kernel_signed_weights(dsa, dtype):
    """Negative and zero weights: (w/2)|s| + (w/2)s must equal w ReLU(s) exactly
    on integer data, including scores that are exactly zero and rank by index."""
    wl = make_prefill(T=600, H=64, d=128, topk=80, dtype=dtype, dist="int", seed=11, w_lo=-3, w_hi=0)
    _prefill_check(dsa, wl, rows=_rows(600, 32, 11))
    wl2 = make_prefill(T=600, H=64, d=128, topk=80, dtype=dtype, dist="int", seed=12)
    wl2.tensors["w"][:, ::2] = 0.0
    _prefill_check(dsa, wl2, rows=_rows(600, 32, 12))
    wl3 = make_prefill(T=500, H=64, d=128, topk=64, dtype=dtype, dist="int", seed=13)
    wl3.tensors["w"] = torch.zeros_like(wl3["w"])  # every score is +0: the lowest indices win
    gi, _ = _prefill_check(dsa, wl3, rows=_rows(500, 16, 13))
    assert (_np(gi)[499] == np.arange(64)).all()


def test_dense_kernel_compaction(dsa):
    """64 heads at d = 128 with K = 16 over 5000 keys: many compactions, with
    non-decreasing scores (every key beats the threshold) and long tie runs."""
    T, H, d, K = 5000, 64, 128, 16
    q = torch.zeros((T, H, d), dtype=torch.float32)
    q[:, 0, 0] = 1.0
    s = torch.arange(T)
    k = torch.zeros((T, d), dtype=torch.float32)
    k[:, 0] = (s // 24 + 1).clamp(max=250).float()
    wl = make_prefill(T=T, H=H, d=d, topk=K, dtype="bf16", dist="int", seed=14)
    w = torch.zeros((T, H))
    w[:, 0] = 1.0
    wl.tensors.update(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), w=w)
    _prefill_check(dsa, wl, rows=_rows(T, 32, 14), exact=True)
    wl2 = make_prefill(T=4000, H=64, d=128, topk=24, dtype="fp8", dist="int", seed=15)
    _prefill_check(dsa, wl2, rows=_rows(4000, 32, 15))


@pytest.mark.parametrize("H,d,dtype,K", [(64, 128, "fp8", 16), (48, 128, "bf16", 40), (8, 32, "bf16", 8),
                                         (16, 64, "fp8", 24)])
def test_compaction_buckets(dsa, H, d, dtype, K):
    """Normal scores, small K over 70000 keys (far more than a candidate
    buffer holds, so the top K streams): most compactions stop after two radix
    digits and keep the K-th best's whole 22-bit key bucket; the final
    selection must still be the exact top K (dense and general kernels)."""
    wl = make_prefill(T=70000, H=H, d=d, topk=K, dtype=dtype, dist="normal", seed=70 + H + K, Tq=192)
    _prefill_check(dsa, wl, rows=_rows(192, 24, 70 + H))


@pytest.mark.parametrize("dtype,dist", [("fp8", "int"), ("bf16", "int"), ("fp8", "normal")])
def test_dense_kernel_streaming_and_full_rows(dsa, dtype, dist):
    """Both top-K modes of the dense kernel: rows of at most 2K + 2048 keys
    (the first 2304 rows of the 6000-key call) keep every score of the row and
    select once at the end; longer rows (the rest of that call, the 40000- and
    70000-key calls) stream their top K through compacting buffers of that
    size; all match the oracle."""
    wl = make_prefill(T=70000, H=64, d=128, topk=100, dtype=dtype, dist=dist, seed=90, Tq=192)
    _prefill_check(dsa, wl, rows=_rows(192, 24, 90))
    short = make_prefill(T=6000, H=64, d=128, topk=100, dtype=dtype, dist=dist, seed=91)
    _prefill_check(dsa, short, rows=_rows(6000, 40, 91))
    mid = make_prefill(T=40000, H=64, d=128, topk=100, dtype=dtype, dist=dist, seed=92, Tq=192)
    _prefill_check(dsa, mid, rows=_rows(192, 24, 92))


def _run_prefill(dsa, wl, K):
    t = {k: v.cuda() for k, v in wl.tensors.items()}
    gi, gs = dsa.indexer_prefill(t["q"], t["k"], t["w"], wl.params["q_pos0"], K, t.get("q_scale"), t.get("k_scale"))
    torch.cuda.synchronize()
    return gi, gs


# Rows of 16K keys and more (E4M3) or 12K and more (bf16) stream from a
# sampled start: one round of the ring of samples (E4M3 T = 24K, bf16 T = 16K,
# K = 2048), two rounds (E4M3 T = 40K, bf16 T = 20K, K = 512), and a call
# whose rows straddle the shortest sampled row, so that workgroups with and
# without a start share the launch.
_SAMPLED = [("fp8", 24576, 2048, 1024, None), ("fp8", 40000, 512, 512, None),
            ("fp8", 17000, 2048, 1024, 16384 - 520),
            ("bf16", 16384, 2048, 1024, None), ("bf16", 20000, 512, 512, None),
            ("bf16", 13000, 2048, 1024, 12288 - 520)]


@pytest.mark.parametrize("dtype,T,K,Tq,q_pos0", _SAMPLED)
@pytest.mark.parametrize("dist", ["normal", "int"])
def test_dense_kernel_sampled_start(dsa, dtype, T, K, Tq, q_pos0, dist):
    """Rows that stream from a sampled start match the oracle (integer inputs
    bit for bit), including the first and last rows of the call."""
    wl = make_prefill(T=T, H=64, d=128, topk=K, dtype=dtype, dist=dist, seed=T % 997 + K, Tq=Tq, q_pos0=q_pos0)
    rows = np.unique(np.concatenate([_rows(Tq, 24, T % 101), [0, 7, 8, Tq - 9, Tq - 1]]))
    _prefill_check(dsa, wl, rows=rows)


@pytest.mark.parametrize("dtype,T,K,Tq,q_pos0", _SAMPLED)
def test_dense_kernel_sampled_start_restream(dsa, monkeypatch, dtype, T, K, Tq, q_pos0):
    """A start that no score beats fails every sampled query's check, so every
    sampled workgroup is streamed again from -inf by the re-stream launch: the
    output is identical to the normal run's, bit for bit, and matches the
    oracle."""
    wl = make_prefill(T=T, H=64, d=128, topk=K, dtype=dtype, dist="normal", seed=T % 991 + K, Tq=Tq,
                      q_pos0=q_pos0)
    a = _run_prefill(dsa, wl, K)
    monkeypatch.setenv("DSAIDX_SAMPLE_RERUN", "1")
    b = _run_prefill(dsa, wl, K)
    monkeypatch.delenv("DSAIDX_SAMPLE_RERUN")
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    monkeypatch.setenv("DSAIDX_SAMPLE_RERUN", "1")
    _prefill_check(dsa, wl, rows=_rows(Tq, 12, T % 89))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_dense_kernel_full_row_edges(dsa, dtype):
    """Full-row top-K at its edges: rows of K - 1, K and K + 1 candidates
    (written whole, or one dropped), and a call where every score is +0, so
    the first digit's bin holds the whole row and the pass that keeps the
    entries at or above it keeps them all; the lowest K indices win."""
    K = 2048
    wl = make_prefill(T=2100, H=64, d=128, topk=K, dtype=dtype, dist="int", seed=95)
    rows = np.unique(np.concatenate([np.arange(K - 3, K + 3), _rows(2100, 10, 95)]))
    _prefill_check(dsa, wl, rows=rows)
    z = make_prefill(T=5000, H=64, d=128, topk=K, dtype=dtype, dist="int", seed=96)
    z.tensors["w"] = torch.zeros_like(z["w"])
    gi, _ = _prefill_check(dsa, z, rows=np.array([0, K - 2, K - 1, K, 3000, 4999]))
    assert (_np(gi)[4999] == np.arange(K)).all()
    assert (_np(gi)[K - 2][: K - 1] == np.arange(K - 1)).all() and (_np(gi)[K - 2][K - 1:] == -1).all()


@pytest.mark.parametrize("Tq,q_pos0,K", [(5, 100, 32), (13, 0, 200), (1, 2047, 2048), (9, 60, 2048)])
def test_dense_kernel_partial_workgroups(dsa, Tq, q_pos0, K):
    """Query counts that leave waves of the first workgroup idle, chunks that
    start mid-sequence, and K at or above the prefix (padding with -1)."""
    wl = make_prefill(T=q_pos0 + Tq, H=64, d=128, topk=K, dtype="fp8", dist="int", seed=Tq + q_pos0,
                      Tq=Tq, q_pos0=q_pos0)
    _prefill_check(dsa, wl)


def test_empty_query_set(dsa):
    wl = make_prefill(T=10, H=4, d=32, topk=4, dtype="bf16", dist="int", seed=11)
    t = {k: v.cuda() for k, v in wl.tensors.items()}
    gi, gs = dsa.indexer_prefill(t["q"][:0], t["k"], t["w"][:0], 0, 4)
    assert gi.shape == (0, 4)


# ------------------------------------------------------------------- decode

def _decode_check(dsa, wl, rows=None, exact=None):
    p = wl.params
    t = {k: v.cuda() for k, v in wl.tensors.items()}
    gi, gs = dsa.indexer_decode(t["q"], t["k_cache"], t["k_scale"], t["w"], t["seq_lens"], p["topk"])
    torch.cuda.synchronize()
    B, N = p["B"], p["N"]
    rows = np.arange(B) if rows is None else np.asarray(rows)
    ri, rs = oracle.decode(wl["q"], wl["k_cache"], wl["k_scale"], wl["w"], wl["seq_lens"], p["topk"], rows=rows)
    exact = (p["dist"] == "int") if exact is None else exact
    kc = wl["k_cache"].reshape(B * N, -1)
    ks = wl["k_scale"].reshape(B * N)

    score_of, cond_of = pair_refs(wl["q"], kc, wl["w"], rows, "bf16", "fp8", None, ks,
                                  key_of=lambda r, keys: rows[r] * N + keys)
    compare(_np(gi)[rows], _np(gs)[rows], ri, rs, exact, score_of, ref_cond_of=cond_of)
    return gi, gs


def test_decode_ragged_exact(dsa):
    lens = [0, 1, 63, 64, 65, 3000, 2999, 1500]
    wl = make_decode(B=8, N=3000, H=64, d=128, topk=64, dist="int", seed=12, seq_lens=lens)
    _decode_check(dsa, wl)


def test_decode_random_tolerance(dsa):
    wl = make_decode(B=4, N=20000, H=64, d=128, topk=2048, dist="normal", seed=13,
                     seq_lens=[20000, 19999, 2048, 2049])
    _decode_check(dsa, wl)


def test_decode_select_paths(dsa):
    """All-equal scores (w = 0: one histogram bin holds the whole row, the exact
    multi-pass path), integer ties at the K-th score (tie cut by index), and a
    cache longer than the select's LDS bitmap."""
    wl = make_decode(B=3, N=20000, H=64, d=128, topk=2048, dist="int", seed=21,
                     seq_lens=[20000, 9000, 2049])
    wl.tensors["w"] = torch.zeros_like(wl["w"])
    gi, gs = _decode_check(dsa, wl)
    assert (_np(gi)[0] == np.arange(2048)).all()
    wl2 = make_decode(B=2, N=30000, H=4, d=64, topk=1000, dist="int", seed=22, seq_lens=[30000, 25000])
    _decode_check(dsa, wl2)
    wl3 = make_decode(B=1, N=600000, H=16, d=64, topk=2048, dist="int", seed=23)
    _decode_check(dsa, wl3)


def test_decode_reused_workspace(dsa):
    """Rows whose first span holds nearly every key (its own K-th best falls in
    the row's threshold bin), decoded with a workspace that a previous call on
    other inputs left full: only the candidates this call gathered may be
    read."""
    lens = [257, 300, 513, 260, 511, 258, 400, 290]
    first = make_decode(B=8, N=600, H=64, d=128, topk=100, dist="int", seed=24, seq_lens=lens)
    wl = make_decode(B=8, N=600, H=64, d=128, topk=100, dist="int", seed=25, seq_lens=lens)
    ws = torch.empty(dsa.workspace_decode(8, 600, 64, 128, 100), dtype=torch.uint8, device="cuda")
    for w in (first, wl):
        t = {k: v.cuda() for k, v in w.tensors.items()}
        gi, gs = dsa.indexer_decode(t["q"], t["k_cache"], t["k_scale"], t["w"], t["seq_lens"], 100, ws=ws)
        torch.cuda.synchronize()
        ri, rs = oracle.decode(w["q"], w["k_cache"], w["k_scale"], w["w"], w["seq_lens"], 100)
        compare(_np(gi), _np(gs), ri, rs, True)


def test_decode_many_rows(dsa):
    """Many short ragged rows (1100 rows of 0 to 300 keys): every row is one
    span, rows of no keys, and rows of at most K keys."""
    lens = [(37 * b) % 301 for b in range(1100)]
    wl = make_decode(B=1100, N=300, H=64, d=128, topk=64, dist="int", seed=15, seq_lens=lens)
    _decode_check(dsa, wl)


def test_decode_rows_of_one_span(dsa):
    """500 ragged rows of one scan span each (0 to 600 keys, top-200): empty
    rows, rows of at most K keys, and rows whose only span's list is the
    whole selection."""
    lens = [(53 * b) % 601 for b in range(500)]
    wl = make_decode(B=500, N=600, H=64, d=128, topk=200, dist="int", seed=16, seq_lens=lens)
    _decode_check(dsa, wl)


def test_decode_lengths_clamped(dsa):
    """Lengths outside [0, Nmax] are clamped on the device: -3 acts as 0 and
    Nmax + 100 as Nmax (the oracle takes the clamped lengths)."""
    wl = make_decode(B=4, N=500, H=64, d=128, topk=64, dist="int", seed=17, seq_lens=[0, 500, 250, 7])
    t = {k: v.cuda() for k, v in wl.tensors.items()}
    lens = torch.tensor([-3, 600, 250, 7], dtype=torch.int32, device="cuda")
    gi, gs = dsa.indexer_decode(t["q"], t["k_cache"], t["k_scale"], t["w"], lens, 64)
    torch.cuda.synchronize()
    ri, rs = oracle.decode(wl["q"], wl["k_cache"], wl["k_scale"], wl["w"], wl["seq_lens"], 64)
    compare(_np(gi), _np(gs), ri, rs, True)


def test_decode_small_heads(dsa):
    wl = make_decode(B=3, N=777, H=7, d=64, topk=100, dist="int", seed=14, seq_lens=[777, 100, 99])
    _decode_check(dsa, wl)


# --------------------------------------------------------------- group bank

def _group_check(dsa, wl, flags=0, rows=None, exact=None):
    p = wl.params
    G, P, K = p["G"], p["P"], p["topk"]
    t = {k: v.cuda() for k, v in wl.tensors.items()}
    pool = bool(flags & dsa.POOL_MEAN)
    gqbar, gwbar = (None, None) if pool else (t["qbar"], t["wbar"])
    gi, gs, gb = dsa.indexer_group_bank(t["q"], t["k"], t["w"], gqbar, gwbar, p["q_pos0"], G, P, K,
                                        t.get("q_scale"), t.get("k_scale"), t.get("qbar_scale"), flags=flags,
                                        want_bank=True)
    torch.cuda.synchronize()
    Tq = p["Tq"]
    rows = np.arange(Tq) if rows is None else np.asarray(rows)
    ri, rs, rb, pairs = oracle.group_bank(wl["q"], wl["k"], wl["w"], wl["qbar"], wl["wbar"], wl.dtype,
                                          p["q_pos0"], G, P, K, flags, wl.tensors.get("q_scale"),
                                          wl.tensors.get("k_scale"), wl.tensors.get("qbar_scale"), rows=rows,
                                          want_bank=True)
    exact = (p["dist"] == "int") if exact is None else exact
    assert pairs == dsa.indexer_group_bank_pairs(Tq, p["q_pos0"], G, P, flags)
    if exact:
        groups = np.unique(rows // G)  # the oracle computes the banks of the requested rows' groups
        assert np.array_equal(_np(gb)[groups], rb[groups])

    score_of, cond_of = pair_refs(wl["q"], wl["k"], wl["w"], rows, wl.dtype, wl.dtype, wl.tensors.get("q_scale"),
                                  wl.tensors.get("k_scale"))
    if exact:
        compare(_np(gi)[rows], _np(gs)[rows], ri, rs, True)
    else:
        # the bank is itself a top-P selection: compare it under the tolerance
        # rule of the group score (Eq. (8)), then compare the rows whose bank
        # is the oracle's bank
        groups = np.unique(rows // G)
        gbank = _np(gb)[groups]
        qbar, wbar = wl["qbar"], wl["wbar"]
        if pool:  # the group score of the pooled query (the oracle's pooling)
            pq, pw = oracle.pool_mean_bf16(wl["q"], wl["w"], G)
            qbar = torch.from_numpy(pq.view(np.int16)).view(torch.bfloat16)
            wbar = torch.from_numpy(pw)
        bscore = np.full(rb[groups].shape, -np.inf)
        for n, g in enumerate(groups):
            v = rb[g][rb[g] >= 0]
            if len(v):
                bscore[n, :len(v)] = oracle.score_pairs(qbar, wl["k"], wbar, np.full(len(v), g), v,
                                                        wl.dtype, wl.dtype, wl.tensors.get("qbar_scale"),
                                                        wl.tensors.get("k_scale"))

        bank_score_of, bank_cond_of = pair_refs(qbar, wl["k"], wbar, groups, wl.dtype, wl.dtype,
                                                wl.tensors.get("qbar_scale"), wl.tensors.get("k_scale"))
        compare(gbank, None, rb[groups], bscore, False, bank_score_of, label="bank", ref_cond_of=bank_cond_of)
        same_bank = np.array([np.array_equal(_np(gb)[r // G], rb[r // G]) for r in rows])
        assert same_bank.mean() > 0.5
        sel = np.nonzero(same_bank)[0]
        compare(_np(gi)[rows][sel], _np(gs)[rows][sel], ri[sel], rs[sel], False,
                lambda r, keys: score_of(sel[r], keys), ref_cond_of=lambda r, keys: cond_of(sel[r], keys))
    return gi, gs, gb


@pytest.mark.parametrize("flags", [0, 1])
def test_group_bank_exact(dsa, flags):
    """Integer inputs, G=4, P=96, K=40, with fallback groups, bank groups and a
    trailing incomplete group."""
    wl = make_group_bank(T=700, H=8, Hs=5, d=32, topk=40, G=4, P=96, dtype="bf16", dist="int", seed=15,
                         Tq=646, q_pos0=52)
    _group_check(dsa, wl, flags)


@pytest.mark.parametrize("G", [8, 16])
def test_group_bank_h64_exact(dsa, G):
    wl = make_group_bank(T=1600, H=64, Hs=64, d=128, topk=128, G=G, P=512, dtype="bf16", dist="int",
                         seed=16 + G)
    _group_check(dsa, wl, rows=_rows(1600, 48, G))


def test_group_bank_fp8_exact(dsa):
    wl = make_group_bank(T=900, H=64, Hs=16, d=128, topk=64, G=16, P=256, dtype="fp8", dist="int", seed=18)
    _group_check(dsa, wl, rows=_rows(900, 48, 18))


@pytest.mark.parametrize("dtype,G,P,K,flags", [("fp8", 8, 200, 96, 1), ("bf16", 16, 77, 40, 1), ("fp8", 8, 130, 96, 0)])
def test_group_bank_dense_gather_exact(dsa, dtype, G, P, K, flags):
    """Bank refinement on the dense kernel (48 heads, d = 128, G a multiple of
    8): banks shorter than a tile and ragged across tiles, forced banks whose
    anchors see fewer than P keys, q_pos0 > 0 and a trailing incomplete group."""
    wl = make_group_bank(T=1300, H=48, Hs=24, d=128, topk=K, G=G, P=P, dtype=dtype, dist="int", seed=60 + G,
                         Tq=1251, q_pos0=48)
    _group_check(dsa, wl, flags, rows=np.unique(np.r_[np.arange(0, 80), _rows(1251, 40, 60 + G), 1250]))


@pytest.mark.parametrize("G", [4, 8, 16])
def test_group_bank_pooled_exact(dsa, G):
    """Training-free group query (mean pooling) at H = 64, d = 128 on integer
    inputs: the pooled query, the bank and every refined row match exactly."""
    wl = make_group_bank(T=1600, H=64, Hs=64, d=128, topk=128, G=G, P=512, dtype="bf16", dist="int",
                         seed=40 + G)
    _group_check(dsa, wl, flags=dsa.POOL_MEAN, rows=_rows(1600, 48, 40 + G))


@pytest.mark.parametrize("flags", [2, 3])
def test_group_bank_pooled_small_heads(dsa, flags):
    """Pooling with the general kernel (8 heads, d = 32), fallback and bank
    groups, a trailing incomplete group and q_pos0 > 0; with and without
    forced banks."""
    wl = make_group_bank(T=700, H=8, Hs=8, d=32, topk=40, G=4, P=96, dtype="bf16", dist="int", seed=44,
                         Tq=646, q_pos0=52)
    _group_check(dsa, wl, flags)


# The group scan's anchor rows (K = P) stream from a sampled start too: rows
# of 12K keys and more (bf16) or 16K and more (E4M3) whose 3.5 P best keys
# lie inside the row.
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("restream", [False, True])
def test_group_scan_sampled_start(dsa, monkeypatch, dtype, restream):
    """Banks of anchors past the shortest sampled row, and the rows refined
    in them, match the oracle bit for bit on integer inputs; also when every
    sampled start is made to fail, so that the re-stream launch builds the
    banks."""
    if restream:
        monkeypatch.setenv("DSAIDX_SAMPLE_RERUN", "1")
    wl = make_group_bank(T=20000, H=64, Hs=48, d=128, topk=256, G=16, P=1024, dtype=dtype, dist="int", seed=70)
    rows = np.unique(np.r_[_rows(20000, 40, 70), 12287, 12288, 16383, 16384, 19999])
    _group_check(dsa, wl, rows=rows)


def test_group_bank_pooled_random(dsa):
    wl = make_group_bank(T=2000, H=64, Hs=64, d=128, topk=256, G=16, P=1024, dtype="bf16", dist="normal",
                         seed=45)
    _group_check(dsa, wl, flags=dsa.POOL_MEAN, rows=_rows(2000, 48, 45))


@pytest.mark.parametrize("G", [4, 8, 16])
def test_pool_mean_kernel_bits(dsa, G):
    """The training-free group query itself, bit for bit: with out_bank given,
    the call keeps the pooled q-bar [groups, H, d] bf16 and w-bar [groups, H]
    fp32 at the start of its workspace (each region 256-byte aligned).  Normal
    inputs, with group 0's first element built so that its mean lies just
    above a bf16 midpoint: members 2, 1 x (G - 3), 1 + G/256 and 2^-27 have the
    mean 1 + 2^-8 + 2^-27/G, which an fp32 sum would put on the midpoint
    1 + 2^-8 (then rounded to even, 1.0); the correctly rounded mean is
    1 + 2^-7.  Every element must equal the oracle's correctly rounded mean."""
    T, H, d, P, K = G * 40 + 5, 64, 128, 64, 16
    wl = make_group_bank(T=T, H=H, Hs=H, d=d, topk=K, G=G, P=P, dtype="bf16", dist="normal", seed=80 + G)
    q, w = wl["q"].clone(), wl["w"].clone()
    members = [2.0] + [1.0] * (G - 3) + [1.0 + G / 256, 2.0 ** -27]
    q[0:G, 0, 0] = torch.tensor(members, dtype=torch.float32).to(torch.bfloat16)
    nfull = T // G
    qb_bytes = -(-nfull * H * d * 2 // 256) * 256
    ws = torch.zeros(dsa.workspace_group_bank(T, T, H, H, d, G, P, K, dsa.DSAIDX_BF16,
                                              dsa.POOL_MEAN | dsa.FORCE_BANK) // 4 + 1,
                     dtype=torch.int32, device="cuda")
    dev = {"q": q.cuda(), "k": wl["k"].cuda(), "w": w.cuda()}
    dsa.indexer_group_bank(dev["q"], dev["k"], dev["w"], None, None, 0, G, P, K,
                           flags=dsa.POOL_MEAN | dsa.FORCE_BANK, want_bank=True, ws=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy().view(np.uint8)
    gq = raw[:nfull * H * d * 2].view(np.uint16).reshape(nfull, H, d)
    gw = raw[qb_bytes:qb_bytes + nfull * H * 4].view(np.float32).reshape(nfull, H)
    rq, rw = oracle.pool_mean_bf16(q, w, G)
    assert np.array_equal(gq, rq[:nfull])
    assert np.array_equal(gw.view(np.uint32), rw[:nfull].view(np.uint32))
    assert gq[0, 0, 0] == 0x3F81


def test_group_bank_random(dsa):
    wl = make_group_bank(T=2000, H=64, Hs=64, d=128, topk=256, G=16, P=1024, dtype="bf16", dist="normal",
                         seed=19)
    _group_check(dsa, wl, rows=_rows(2000, 48, 19))


# ------------------------------------------------------- MTP verification

def _mtp_check(dsa, wl, flags=0, rows=None, exact=None, lens_dev=None):
    p = wl.params
    B, N, m, G, P, K = p["B"], p["N"], p["m"], p["G"], p["P"], p["topk"]
    t = {k: v.cuda() for k, v in wl.tensors.items()}
    pool = bool(flags & dsa.POOL_MEAN)
    lens = t["prefix_lens"] if lens_dev is None else torch.as_tensor(lens_dev, dtype=torch.int32).cuda()
    gi, gs, gb = dsa.indexer_mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], None if pool else t["qbar"],
                                 None if pool else t["wbar"], lens, G, P, K, flags=flags, want_bank=True)
    torch.cuda.synchronize()
    gi, gs, gb = _np(gi).reshape(B * m, K), _np(gs).reshape(B * m, K), _np(gb)
    rows = np.arange(B * m) if rows is None else np.asarray(rows)
    ri, rs, rb, _ = oracle.mtp(wl["q"], wl["k_cache"], wl["k_scale"], wl["w"], wl["qbar"], wl["wbar"],
                               wl["prefix_lens"], G, P, K, flags=flags, rows=rows, want_bank=True)
    exact = (p["dist"] == "int") if exact is None else exact
    qf = wl["q"].reshape(B * m, p["H"], p["d"])
    wf = wl["w"].reshape(B * m, p["H"])
    kc = wl["k_cache"].reshape(B * N, -1)
    ks = wl["k_scale"].reshape(B * N)
    if pool:
        pooled = [oracle.pool_mean_bf16(wl["q"][b], wl["w"][b], G) for b in range(B)]
        qbar = torch.from_numpy(np.stack([x[0] for x in pooled]).view(np.int16)).view(torch.bfloat16)
        wbar = torch.from_numpy(np.stack([x[1] for x in pooled]))
    else:
        qbar, wbar = wl["qbar"], wl["wbar"]
    NGs = m // G
    qbf = qbar.reshape(B * NGs, -1, p["d"])
    wbf = wbar.reshape(B * NGs, -1)
    if exact:
        assert np.array_equal(gb, rb), "banks differ"
        compare(gi[rows], gs[rows], ri, rs, True)
        return gi, gs, gb
    # banks under the tolerance rule of the group score, then the rows whose
    # bank is the oracle's
    for b in range(B):
        for g in range(NGs):
            v = rb[b, g][rb[b, g] >= 0]
            if len(v) == 0:
                assert (gb[b, g] == -1).all()
                continue
            grp = b * NGs + g

            bank_score, bank_cond = pair_refs(qbf, kc, wbf, [grp], "bf16", "fp8", None, ks,
                                              key_of=lambda r, keys, b=b: b * N + keys)
            compare(gb[b, g][None], None, rb[b, g][None], bank_score(0, v)[None], False, bank_score,
                    label=f"bank {b},{g}", ref_cond_of=bank_cond)

    score_of, cond_of = pair_refs(qf, kc, wf, rows, "bf16", "fp8", None, ks,
                                  key_of=lambda r, keys: (rows[r] // m) * N + keys)
    same = np.array([np.array_equal(gb[r // m, (r % m) // G], rb[r // m, (r % m) // G]) for r in rows])
    assert same.mean() > 0.5
    sel = np.nonzero(same)[0]
    compare(gi[rows][sel], gs[rows][sel], ri[sel], rs[sel], False, lambda r, keys: score_of(sel[r], keys),
            ref_cond_of=lambda r, keys: cond_of(sel[r], keys))
    return gi, gs, gb


@pytest.mark.parametrize("G", [4, 8, 16])
def test_mtp_mixed_windows_exact(dsa, G):
    """Integer inputs, 64-head queries, a 16-head group indexer; windows that
    fall back (N << P, N == P) and windows that share banks (N == P+1, N at the
    end of the cache)."""
    P = 256
    wl = make_mtp(B=4, N=3000, m=16, H=64, Hs=16, d=128, topk=64, G=G, P=P, dist="int", seed=50 + G,
                  prefix_lens=[40, P, P + 1, 3000 - 16 + 1])
    gi, _, gb = _mtp_check(dsa, wl)
    assert (gb[:2] == -1).all() and (gb[2:] >= 0).all()


@pytest.mark.parametrize("G,m,d", [(8, 16, 128), (4, 16, 128), (4, 32, 128), (4, 16, 64)])
def test_mtp_shared_anchor_scan(dsa, G, m, d):
    """An 8-head group indexer: the 2 or 4 anchors of a window (or of half a
    window, m = 32) are scored in one pass over the cache.  Their lengths
    differ by G keys, windows that fall back have no anchor keys, and the
    banks and every refined row match exactly on integer inputs."""
    P = 256
    wl = make_mtp(B=4, N=3000, m=m, H=64, Hs=8, d=d, topk=64, G=G, P=P, dist="int", seed=80 + G + m + d,
                  prefix_lens=[40, P + 1, 1700, 3000 - m + 1])
    gi, _, gb = _mtp_check(dsa, wl)
    assert (gb[:1] == -1).all() and (gb[1:] >= 0).all()


def test_mtp_shared_anchor_block_edges(dsa):
    """Anchors of one window that end on either side of a 256-key scan span
    boundary (lengths 256 and 264, 512 and 520, 767 and 775): the workgroup
    scores a span for one of its rows and not for the other."""
    wl = make_mtp(B=3, N=1200, m=16, H=64, Hs=8, d=128, topk=64, G=8, P=255, dist="int", seed=91,
                  prefix_lens=[256, 512, 767])
    _, _, gb = _mtp_check(dsa, wl)
    assert (gb >= 0).any(axis=-1).all()


def test_mtp_pooled_exact(dsa):
    wl = make_mtp(B=3, N=5000, m=16, H=64, Hs=64, d=128, topk=128, G=8, P=1024, dist="int", seed=54,
                  prefix_lens=[1500, 4985, 900])
    _mtp_check(dsa, wl, flags=dsa.POOL_MEAN)


def test_mtp_small_heads_d64(dsa):
    """General shapes: 8 heads at d = 64, a 4-head group indexer, topk == P."""
    wl = make_mtp(B=5, N=700, m=8, H=8, Hs=4, d=64, topk=48, G=4, P=48, dist="int", seed=55,
                  prefix_lens=[1, 47, 48, 49, 693])
    _mtp_check(dsa, wl)


def test_mtp_prefix_clamped(dsa):
    """Prefix lengths outside [1, Nmax-m+1] act as the nearest bound."""
    wl = make_mtp(B=3, N=600, m=16, H=16, Hs=8, d=128, topk=32, G=4, P=100, dist="int", seed=56,
                  prefix_lens=[1, 585, 585])
    _mtp_check(dsa, wl, lens_dev=[-5, 585, 100000])


def test_mtp_random_tolerance(dsa):
    wl = make_mtp(B=4, N=20000, m=16, H=64, Hs=16, d=128, topk=512, G=4, P=2048, dist="normal", seed=57,
                  prefix_lens=[19985, 12000, 2048, 5000])
    _mtp_check(dsa, wl, rows=_rows(64, 40, 57))


def test_mtp_no_bank_is_dense(dsa):
    """NO_BANK: every window uses the original indexer, eligible or not."""
    wl = make_mtp(B=3, N=4000, m=16, H=64, Hs=8, d=128, topk=256, G=8, P=512, dist="int", seed=58,
                  prefix_lens=[3985, 100, 2000])
    _, _, gb = _mtp_check(dsa, wl, flags=dsa.NO_BANK)
    assert (gb == -1).all()



# ------------------------------------------------------- calibration kernels

def test_union_sizes_and_overlap(dsa):
    """Union sizes of groups of G rows and per-row overlaps against the
    oracle, on random sorted index sets with -1 padding, on sets past the
    first 2^18 tokens (a second bitmap pass), and on real indexer output
    (dense top-K vs the group-bank top-K of the same queries)."""
    import oracle.calib as calib
    rng = np.random.default_rng(7)
    T, K = 96, 300
    idx = np.full((T, K), -1, np.int32)
    for r in range(T):
        n = rng.integers(0, K + 1)
        hi = 600000 if r % 3 == 0 else 5000
        idx[r, :n] = np.sort(rng.choice(hi, size=n, replace=False))
    gi = torch.from_numpy(idx).cuda()
    for G in (4, 8, 16):
        got = dsa.union_sizes(gi, G).cpu().numpy()
        assert np.array_equal(got, calib.union_sizes(idx, G)), G
    other = np.roll(idx, 1, axis=0)
    got = dsa.topk_overlap(gi, torch.from_numpy(other).cuda()).cpu().numpy()
    assert np.array_equal(got, calib.overlap_counts(idx, other))
    wl = make_group_bank(T=2000, H=16, Hs=8, d=64, topk=64, G=8, P=256, dtype="bf16", dist="normal", seed=70)
    t = {k: v.cuda() for k, v in wl.tensors.items()}
    di, _ = dsa.indexer_prefill(t["q"], t["k"], t["w"], 0, 64)
    bi, _, _ = dsa.indexer_group_bank(t["q"], t["k"], t["w"], t["qbar"], t["wbar"], 0, 8, 256, 64)
    u = dsa.union_sizes(di, 8).cpu().numpy()
    assert np.array_equal(u, calib.union_sizes(di.cpu().numpy(), 8))
    cov = dsa.topk_overlap(di, bi).cpu().numpy()
    assert np.array_equal(cov, calib.overlap_counts(di.cpu().numpy(), bi.cpu().numpy()))
    # rows before the first bank group use the original indexer: full coverage
    assert np.array_equal(cov[:256], (di[:256] >= 0).sum(1).cpu().numpy())



# --------------------------------------------------- group query (Eq. 6-7)

@pytest.mark.parametrize("G,Tq,q_pos0,rope_dim,dc,dh,Hs", [(16, 1024, 0, 64, 256, 512, 8),
                                                            (8, 1003, 40960, 64, 256, 512, 8),
                                                            (4, 64, 131000, 128, 256, 512, 8),
                                                            (16, 40, 7, 0, 256, 512, 8),
                                                            (4, 2100, 96, 64, 80, 48, 3)])
def test_group_query(dsa, G, Tq, q_pos0, rope_dim, dc, dh, Hs):
    """qbar and wbar of Eq. (6)-(7) against the oracle: a random pooling
    projection, the rotary part at large anchor positions, an incomplete last
    group; bf16 queries agree within two bf16 steps (almost all exactly).  The
    last case has partial product tiles in every dimension (525 groups, 80 and
    384 columns, k of 240 and 80: partial 64-k chunks)."""
    from oracle import group_query as gq
    d = 128
    g = torch.Generator().manual_seed(80 + G)
    c = torch.randn(Tq, dc, generator=g).to(torch.bfloat16)
    h = torch.randn(Tq, dh, generator=g).to(torch.bfloat16)
    wp = (torch.randn(dc, 3 * dc, generator=g) / (3 * dc) ** 0.5).to(torch.bfloat16)
    wq = (torch.randn(Hs * d, dc, generator=g) / dc ** 0.5).to(torch.bfloat16)
    wg = (torch.randn(Hs, dh, generator=g) / dh ** 0.5).to(torch.bfloat16)
    qb, wb = dsa.indexer_group_query(c.cuda(), h.cuda(), wp.cuda(), wq.cuda(), wg.cuda(), G, Hs, d, q_pos0,
                                     rope_dim)
    torch.cuda.synchronize()
    rq, rw = gq.group_query(c, h, wp, wq, wg, G, Hs, d, q_pos0, rope_dim)
    gqv = qb.double().cpu().numpy()
    scale = np.abs(rq).max(axis=2, keepdims=True) + 1e-30
    assert (np.abs(gqv - rq) <= 2 * 2.0 ** -8 * scale).all()
    assert (gqv == rq).mean() > 0.97
    np.testing.assert_allclose(wb.cpu().numpy(), rw, rtol=0, atol=2e-5)
    if Tq % G:
        assert (qb[-1] == 0).all() and (wb[-1] == 0).all()
