"""Pins for the CPU oracle: what the pages and the mathematics fix, independent of
the oracle's own code.  CPU only.

Each test names the mistake it is there to catch.  References are to
"ADIndex: Layer-Adaptive Sparse Attention Indexing via Group-Level
Distillation" (Qi et al.).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.bruteforce import lexsort_topk
from workloads import make_decode, make_group_bank, make_mtp, make_prefill, to_bf16
from workloads.gen import e4m3_quantize_rows

GOLDEN = __file__.replace("test_oracle_pins.py", "golden/table5_speedups.txt")


def _bf16(x):
    return to_bf16(torch.as_tensor(np.asarray(x, np.float32)))


def _f64(t):
    return t.float().double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def _matmul_topk(qv, kv, q_pos0, K):
    """Library-routine reference for H=1, w=1, q,k >= 0: score = q . k."""
    S = qv @ kv.T
    Tq, Tk = S.shape
    valid = np.arange(Tk)[None, :] <= (q_pos0 + np.arange(Tq))[:, None]
    return lexsort_topk(S, valid, K), S


# ------------------------------------------------------------------ decoders

def test_e4m3_decoder_matches_torch(oracle_lib):
    """All 256 E4M3 codes against torch's float8_e4m3fn (OCP E4M3) conversion."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(ref[~nan], got[~nan])
    assert oracle.e4m3_to_double(0x7E) == 448.0 and oracle.e4m3_to_double(0x01) == 2.0 ** -9


def test_bf16_decoder_matches_torch(oracle_lib):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, 4000)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite patterns
    ref = torch.as_tensor(bits.astype(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    assert np.array_equal(ref, got)


# ----------------------------------------------------------- Eq. (1)-(2) pins

@pytest.mark.parametrize("Tq,Tk,d,K", [(40, 97, 32, 16), (97, 97, 16, 200), (1, 5, 8, 3)])
def test_single_head_is_a_matmul(oracle_lib, Tq, Tk, d, K):
    """H=1, w=1, q,k >= 0: Eq. (1) is q . k.  Checked against np.matmul and a
    full lexsort.  Catches a transposed operand, a wrong ReLU sign, causal or
    q_pos0 off-by-ones, the tie rule and the padding."""
    rng = np.random.default_rng(Tq * 131 + Tk)
    qv = rng.integers(0, 4, (Tq, 1, d)).astype(np.float32)
    kv = rng.integers(0, 4, (Tk, d)).astype(np.float32)
    q_pos0 = Tk - Tq
    idx, sc = oracle.prefill(_bf16(qv), _bf16(kv), np.ones((Tq, 1), np.float32), "bf16", q_pos0, K)
    (ref_i, ref_s), _ = _matmul_topk(qv[:, 0, :].astype(np.float64), kv.astype(np.float64), q_pos0, K)
    assert np.array_equal(idx, ref_i)
    assert np.array_equal(sc, ref_s)


def test_one_hot_keys_known_ranking(oracle_lib):
    """Key s is c_s times the unit vector e_{s mod d} and every query entry is
    1, so every head's dot product is c_s: the score is c_s * sum_j w_j where
    c_s > 0 and 0 otherwise (ReLU), whatever the sign of the weights' sum.
    The ranking follows c_s (ties by index) for a positive weight sum and
    puts the zero scores first for a negative one."""
    T, H, d, K = 60, 3, 8, 10
    rng = np.random.default_rng(11)
    cs = rng.integers(-3, 4, T).astype(np.float64)
    k = np.zeros((T, d))
    k[np.arange(T), np.arange(T) % d] = cs
    q = np.ones((T, H, d))
    for wsum_sign in (1, -1):
        w = np.full((T, H), 0.5 * wsum_sign)
        idx, sc = oracle.prefill(_bf16(q), _bf16(k), w.astype(np.float32), "bf16", 0, K)
        want = np.maximum(cs, 0) * w[0].sum()  # the same weights for every query
        for t in (0, 9, 59):
            valid = np.arange(T) <= t
            ri, rs = lexsort_topk(want[None, :], valid[None, :], K)
            assert np.array_equal(idx[t], ri[0]) and np.array_equal(sc[t], rs[0]), (wsum_sign, t)


def test_relu_acts_per_head(oracle_lib):
    """Heads q and -q with unit weights: ReLU(x) + ReLU(-x) = |x|.  A dropped
    ReLU gives 0, a ReLU after the head sum gives 0."""
    rng = np.random.default_rng(2)
    Tq = Tk = 64
    d = 16
    q0 = rng.integers(-3, 4, (Tq, d)).astype(np.float32)
    kv = rng.integers(-3, 4, (Tk, d)).astype(np.float32)
    q = np.stack([q0, -q0], axis=1)
    idx, sc = oracle.prefill(_bf16(q), _bf16(kv), np.ones((Tq, 2), np.float32), "bf16", 0, 8)
    S = np.abs(q0.astype(np.float64) @ kv.T.astype(np.float64))
    ref_i, ref_s = lexsort_topk(S, np.tril(np.ones((Tq, Tk), bool)), 8)
    assert np.array_equal(idx, ref_i) and np.array_equal(sc, ref_s)


def test_gate_weights_scale_their_own_head(oracle_lib):
    """q_j = c_j q_0 with c_j > 0: the score is (sum_j w_{t,j} c_j) ReLU(q_0 . k),
    with per-query, per-head w of mixed sign.  Catches a w indexed by the wrong
    query or head, and a transposed [H,d] layout."""
    rng = np.random.default_rng(3)
    Tq, Tk, d, H = 30, 50, 8, 3
    c = np.array([1.0, 2.0, 0.5])
    q0 = rng.integers(-3, 4, (Tq, d)).astype(np.float32)
    q = q0[:, None, :] * c[None, :, None]
    w = rng.integers(-3, 4, (Tq, H)).astype(np.float32)
    kv = rng.integers(-3, 4, (Tk, d)).astype(np.float32)
    q_pos0 = Tk - Tq
    idx, sc = oracle.prefill(_bf16(q.astype(np.float32)), _bf16(kv), w, "bf16", q_pos0, Tk)
    coef = (w.astype(np.float64) * c[None, :]).sum(1)
    S = coef[:, None] * np.maximum(q0.astype(np.float64) @ kv.T.astype(np.float64), 0.0)
    valid = np.arange(Tk)[None, :] <= (q_pos0 + np.arange(Tq))[:, None]
    ref_i, ref_s = lexsort_topk(S + 0.0, valid, Tk)
    assert np.array_equal(idx, ref_i)
    assert np.array_equal(sc, ref_s)


def test_zero_weights_rank_by_index(oracle_lib):
    """w = 0: every score is 0 (and -0 ranks as +0), so the selection is the
    first min(K, t+1) positions."""
    wl = make_prefill(T=70, H=4, d=16, topk=32, dtype="bf16", dist="int", seed=4)
    w = -np.zeros((70, 4), np.float32)
    idx, sc = oracle.prefill(wl["q"], wl["k"], w, "bf16", 0, 32)
    for t in range(70):
        m = min(32, t + 1)
        assert list(idx[t, :m]) == list(range(m)) and (idx[t, m:] == -1).all()
        assert (sc[t, :m] == 0).all() and np.isneginf(sc[t, m:]).all()


def test_bruteforce_random_small(oracle_lib):
    """The full score matrix (numpy einsum) then a full lexsort per row, on
    integer inputs with many ties; several heads, K above and below the prefix."""
    for seed, (T, H, d, K) in enumerate([(96, 4, 32, 16), (50, 3, 8, 64), (130, 5, 16, 33)]):
        wl = make_prefill(T=T, H=H, d=d, topk=K, dtype="bf16", dist="int", seed=seed)
        q = _f64(wl["q"])
        k = _f64(wl["k"])
        w = _f64(wl["w"])
        S = (w[:, :, None] * np.maximum(np.einsum("thc,sc->ths", q, k), 0)).sum(1)
        ref_i, ref_s = lexsort_topk(S, np.tril(np.ones((T, T), bool)), K)
        idx, sc = oracle.prefill(wl["q"], wl["k"], wl["w"], "bf16", 0, K)
        assert np.array_equal(idx, ref_i) and np.array_equal(sc, ref_s)


def test_invariants_and_rows(oracle_lib):
    """Selected indices are causal, distinct, ascending, exactly min(K, t+1);
    computing a subset of rows gives the same rows."""
    wl = make_prefill(T=300, H=4, d=32, topk=40, dtype="bf16", dist="normal", seed=5, Tq=120)
    q_pos0 = wl.params["q_pos0"]
    idx, sc = oracle.prefill(wl["q"], wl["k"], wl["w"], "bf16", q_pos0, 40)
    for i in range(120):
        t = q_pos0 + i
        v = idx[i][idx[i] >= 0]
        assert len(v) == min(40, t + 1) and (np.diff(v) > 0).all() and v.max() <= t
    rows = [0, 7, 119, 7]
    i2, s2 = oracle.prefill(wl["q"], wl["k"], wl["w"], "bf16", q_pos0, 40, rows=rows)
    assert np.array_equal(i2, idx[rows]) and np.array_equal(s2, sc[rows])


def test_fp8_scales_multiply_each_token(oracle_lib):
    """E4M3 inputs with per-token scales, H=1, w=1, non-negative values: the
    score is the matmul of the torch-dequantised tensors."""
    rng = np.random.default_rng(6)
    Tq = Tk = 48
    d = 32
    qf = torch.as_tensor(np.abs(rng.standard_normal((Tq, 1, d))).astype(np.float32))
    kf = torch.as_tensor(np.abs(rng.standard_normal((Tk, d))).astype(np.float32) * 5)
    qc, qs = e4m3_quantize_rows(qf.reshape(Tq, d))
    kc, ks = e4m3_quantize_rows(kf)
    idx, sc = oracle.prefill(qc.reshape(Tq, 1, d), kc, np.ones((Tq, 1), np.float32), "fp8", 0, 10,
                             q_scale=qs, k_scale=ks)
    qd = qc.view(torch.float8_e4m3fn).double() * qs.double()[:, None]
    kd = kc.view(torch.float8_e4m3fn).double() * ks.double()[:, None]
    S = (qd @ kd.T).numpy()
    ref_i, ref_s = lexsort_topk(S, np.tril(np.ones((Tq, Tk), bool)), 10)
    assert np.array_equal(idx, ref_i)
    np.testing.assert_allclose(sc, ref_s, rtol=1e-14)


# ------------------------------------------------------------------- decode

def test_decode_equals_prefill_row(oracle_lib):
    """decode with seq_len = t+1 is prefill row t (integer values: the E4M3 cache
    converts exactly to the bf16 keys of the prefill call); ragged lengths."""
    B, N, H, d, K = 5, 90, 4, 32, 20
    lens = [90, 1, 37, 64, 20]
    wl = make_decode(B, N, H, d, K, dist="int", seed=7, seq_lens=lens)
    idx, sc = oracle.decode(wl["q"], wl["k_cache"], wl["k_scale"], wl["w"], wl["seq_lens"], K)
    kb = to_bf16(wl["k_cache"].view(torch.float8_e4m3fn).float())
    for b in range(B):
        n = lens[b]
        pi, ps = oracle.prefill(wl["q"][b:b + 1], kb[b, :n], wl["w"][b:b + 1], "bf16", n - 1, K)
        assert np.array_equal(idx[b], pi[0]) and np.array_equal(sc[b], ps[0])


def test_decode_single_head_matmul(oracle_lib):
    B, N, d, K = 3, 200, 64, 50
    rng = np.random.default_rng(8)
    q = np.abs(rng.standard_normal((B, 1, d))).astype(np.float32)
    kf = torch.as_tensor(np.abs(rng.standard_normal((B * N, d))).astype(np.float32))
    kc, ks = e4m3_quantize_rows(kf)
    qb = _bf16(q)
    idx, sc = oracle.decode(qb, kc.reshape(B, N, d), ks.reshape(B, N), np.ones((B, 1), np.float32),
                            np.array([200, 150, 3], np.int32), K)
    kd = (kc.view(torch.float8_e4m3fn).double() * ks.double()[:, None]).numpy().reshape(B, N, d)
    for b, n in enumerate([200, 150, 3]):
        S = (qb[b].double().numpy() @ kd[b, :n].T)
        ri, rs = lexsort_topk(S, np.ones_like(S, bool), K)
        assert np.array_equal(idx[b], ri[0])
        np.testing.assert_allclose(sc[b], rs[0], rtol=1e-14)


# ------------------------------------------------- single-pair scores, Eq. (1)

def test_score_pairs_single_head_is_a_matmul(oracle_lib):
    """H=1, w=1, q,k >= 0: the score of pair (row r, key s) is q_r . k_s.
    Checked against np.matmul on a query array and a key array of different
    lengths, at pairs whose row and key differ: catches a w or q row taken
    from the key index, a key row taken from the query index, and a
    transposed operand."""
    rng = np.random.default_rng(40)
    Tq, Tk, d = 23, 61, 32
    qv = rng.integers(0, 4, (Tq, 1, d)).astype(np.float32)
    kv = rng.integers(0, 4, (Tk, d)).astype(np.float32)
    rows = rng.integers(0, Tq, 300)
    keys = rng.integers(0, Tk, 300)
    got = oracle.score_pairs(_bf16(qv), _bf16(kv), np.ones((Tq, 1), np.float32), rows, keys, "bf16", "bf16")
    S = np.matmul(qv[:, 0, :].astype(np.float64), kv.T.astype(np.float64))
    assert np.array_equal(got, S[rows, keys])


def _pairs_of(idx):
    r, c = np.nonzero(idx >= 0)
    return r, idx[r, c], c


@pytest.mark.parametrize("dtype,gates", [("bf16", "mixed"), ("bf16", "negative"), ("fp8", "mixed"),
                                         ("fp8", "negative")])
def test_score_pairs_equal_prefill_scores(oracle_lib, dtype, gates):
    """Every selected (row, key) of a dense prefill call, rescored one pair at
    a time, gives the score the prefill call reported for it (bf16, and E4M3
    with per-token scales; queries at q_pos0 > 0 so a row is not its position;
    gates of mixed sign, or all negative as w = -|N(0,1)|/8).  The prefill
    scores are pinned by the brute-force and closed-form tests above, so a
    wrong w row, a dropped or misapplied scale, or a swapped dtype code in the
    pair scorer fails here."""
    T, Tq, H, d, K = 150, 60, 6, 32, 40
    wl = make_prefill(T=T, H=H, d=d, topk=K, dtype=dtype, dist="normal", seed=41, Tq=Tq)
    w = wl["w"].numpy()
    if gates == "negative":
        w = -np.abs(np.random.default_rng(42).standard_normal((Tq, H))).astype(np.float32) / 8
    q_pos0 = wl.params["q_pos0"]
    qs, ks = wl.tensors.get("q_scale"), wl.tensors.get("k_scale")
    idx, sc = oracle.prefill(wl["q"], wl["k"], w, dtype, q_pos0, K, qs, ks)
    r, keys, c = _pairs_of(idx)
    got = oracle.score_pairs(wl["q"], wl["k"], w, r, keys, dtype, dtype, qs, ks)
    assert np.array_equal(got, sc[r, c])
    if gates == "negative":  # every term is w * ReLU(.) <= 0
        assert (got <= 0).all()


def test_score_pairs_decode_layout(oracle_lib):
    """The decode layout: bf16 queries [B,H,d] against an E4M3 cache passed
    flattened to [B*N, d] with its scales [B*N]; pair (b, b*N + s) is key s of
    sequence b.  It must give the decode call's reported scores (pinned by
    decode == prefill row above): catches swapped q/k dtype codes and a wrong
    flattened cache index."""
    B, N, H, d, K = 4, 120, 8, 64, 30
    lens = [120, 77, 5, 64]
    wl = make_decode(B, N, H, d, K, dist="normal", seed=43, seq_lens=lens)
    idx, sc = oracle.decode(wl["q"], wl["k_cache"], wl["k_scale"], wl["w"], wl["seq_lens"], K)
    b, keys, c = _pairs_of(idx)
    kc = wl["k_cache"].reshape(B * N, d)
    ks = wl["k_scale"].reshape(B * N)
    got = oracle.score_pairs(wl["q"], kc, wl["w"], b, b * N + keys, "bf16", "fp8", None, ks)
    assert np.array_equal(got, sc[b, c])
    # the same pairs through torch's E4M3 decoder and a numpy Eq. (1)
    qd = wl["q"].double().numpy()
    kd = (kc.view(torch.float8_e4m3fn).double() * ks.double()[:, None]).numpy()
    dots = np.einsum("phc,pc->ph", qd[b], kd[b * N + keys])
    ref = (wl["w"].double().numpy()[b] * np.maximum(dots, 0.0)).sum(1)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-300)


def test_score_pairs_cond_closed_forms(oracle_lib):
    """The absolute condition of Eq. (1), C = sum_j |w_j| sum_c |q_jc| |k_c|:
    with H = 1 and |w| = 1 it is |q| @ |k|^T (np.matmul of the magnitudes,
    whatever the signs); with non-negative q, k, w every ReLU and |.| is the
    identity, so C equals the pinned pair score exactly (bf16, and E4M3 with
    per-token scales); for signed inputs C >= |score|, and w = 0 gives 0."""
    rng = np.random.default_rng(44)
    Tq, Tk, d = 17, 40, 32
    qv = rng.integers(-3, 4, (Tq, 1, d)).astype(np.float32)
    kv = rng.integers(-3, 4, (Tk, d)).astype(np.float32)
    w = np.where(rng.random((Tq, 1)) < 0.5, -1.0, 1.0).astype(np.float32)
    rows, keys = rng.integers(0, Tq, 200), rng.integers(0, Tk, 200)
    got = oracle.score_pairs_cond(_bf16(qv), _bf16(kv), w, rows, keys, "bf16", "bf16")
    ref = np.matmul(np.abs(qv[:, 0, :]).astype(np.float64), np.abs(kv).T.astype(np.float64))
    assert np.array_equal(got, ref[rows, keys])
    for dtype in ("bf16", "fp8"):
        wl = make_prefill(T=90, H=5, d=64, topk=8, dtype=dtype, dist="int", seed=45)
        q, k = wl["q"], wl["k"]
        if dtype == "bf16":
            q, k = _bf16(np.abs(_f64(q))), _bf16(np.abs(_f64(k)))
            qs = ks = None
        else:
            qf = torch.as_tensor(np.abs(rng.standard_normal((90, 5 * 64))).astype(np.float32))
            kf = torch.as_tensor(np.abs(rng.standard_normal((90, 64))).astype(np.float32))
            q, qs = e4m3_quantize_rows(qf)
            k, ks = e4m3_quantize_rows(kf)
            q = q.reshape(90, 5, 64)
        wn = np.abs(rng.standard_normal((90, 5))).astype(np.float32)
        r2, k2 = rng.integers(0, 90, 300), rng.integers(0, 90, 300)
        c = oracle.score_pairs_cond(q, k, wn, r2, k2, dtype, dtype, qs, ks)
        sc = oracle.score_pairs(q, k, wn, r2, k2, dtype, dtype, qs, ks)
        assert np.array_equal(c, sc), dtype
    wl = make_prefill(T=60, H=8, d=32, topk=8, dtype="bf16", dist="normal", seed=46)
    r3, k3 = rng.integers(0, 60, 300), rng.integers(0, 60, 300)
    c = oracle.score_pairs_cond(wl["q"], wl["k"], wl["w"], r3, k3, "bf16", "bf16")
    sc = oracle.score_pairs(wl["q"], wl["k"], wl["w"], r3, k3, "bf16", "bf16")
    assert (c >= np.abs(sc)).all() and (c > 0).all()
    assert (oracle.score_pairs_cond(wl["q"], wl["k"], np.zeros((60, 8), np.float32), r3, k3, "bf16", "bf16")
            == 0).all()


def test_tolerance_rule_accepts_rounding_rejects_errors(oracle_lib):
    """The comparison rule: perturbing the oracle's scores by binary32-level
    rounding (2^-20 of each key's absolute condition) passes, also on a row
    whose K-th score is near zero; a 2% error on one clearly selected key, a
    dropped key well above the K-th score, or a wrong count fails."""
    from tests.parity import compare, pair_refs
    T, K = 300, 64
    wl = make_prefill(T=T, H=16, d=64, topk=K, dtype="bf16", dist="normal", seed=47)
    rows = np.arange(100, 300, 7)
    ri, rs = oracle.prefill(wl["q"], wl["k"], wl["w"], "bf16", 0, K, rows=rows)
    score_of, cond_of = pair_refs(wl["q"], wl["k"], wl["w"], rows, "bf16", "bf16")
    cond = np.zeros(ri.shape)
    for n in range(len(rows)):
        v = ri[n] >= 0
        cond[n, v] = cond_of(n, ri[n][v])
    rng = np.random.default_rng(48)
    noisy = rs + np.where(ri >= 0, rng.uniform(-1, 1, rs.shape) * 2.0 ** -20 * cond, 0.0)
    compare(ri, noisy, ri, rs, False, score_of, ref_cond_of=cond_of)
    bad = rs.copy()
    n = 3
    top = np.argmax(rs[n])
    bad[n, top] *= 1.02
    with pytest.raises(AssertionError):
        compare(ri, bad, ri, rs, False, score_of, ref_cond_of=cond_of)
    dropped = ri.copy()
    keep = np.delete(dropped[n][dropped[n] >= 0], top)
    dropped[n] = -1
    others = np.setdiff1d(np.arange(rows[n] + 1), ri[n])
    dropped[n][:K] = np.sort(np.concatenate([keep, others[:1]]))
    with pytest.raises(AssertionError):
        compare(dropped, None, ri, rs, False, score_of, ref_cond_of=cond_of)
    short = ri.copy()
    short[n, K - 1] = -1
    with pytest.raises(AssertionError):
        compare(short, None, ri, rs, False, score_of, ref_cond_of=cond_of)


# --------------------------------------------------------- group bank pins

def _gb(T, G, P, K, seed, Hs=None, H=4, d=16, Tq=None, dist="int", **kw):
    return make_group_bank(T=T, H=H, Hs=Hs or H, d=d, topk=K, G=G, P=P, dtype="bf16", dist=dist,
                           seed=seed, Tq=Tq, **kw)


def test_full_bank_equals_dense(oracle_lib):
    """Forced bank with P >= every prefix: the bank is the whole prefix, so
    every query's candidate set is its whole prefix and the result is dense."""
    wl = _gb(T=80, G=4, P=128, K=24, seed=9, Tq=64)
    p = wl.params
    d_i, d_s = oracle.prefill(wl["q"], wl["k"], wl["w"], "bf16", p["q_pos0"], 24)
    g_i, g_s, bank, _ = oracle.group_bank(wl["q"], wl["k"], wl["w"], wl["qbar"], wl["wbar"], "bf16",
                                          p["q_pos0"], 4, 128, 24, flags=oracle.FORCE_BANK,
                                          want_bank=True)
    assert np.array_equal(d_i, g_i) and np.array_equal(d_s, g_s)
    for g in range(16):
        a = p["q_pos0"] + 4 * g
        assert list(bank[g][bank[g] >= 0]) == list(range(a + 1))


def test_anchor_query_as_group_query_recovers_dense(oracle_lib):
    """With q-bar = the anchor's own q and w-bar = its w, and K <= P, the anchor's
    top-K lies inside the bank (a top-P of the same score), so the anchor row
    equals the dense row (the exact-recovery statement of Section 1)."""
    T, G, P, K = 200, 8, 40, 12
    wl = _gb(T=T, G=G, P=P, K=K, seed=10, dist="normal")
    qbar = wl["q"][::G].clone()
    wbar = wl["w"][::G].clone()
    d_i, _ = oracle.prefill(wl["q"], wl["k"], wl["w"], "bf16", 0, K)
    g_i, _, bank, _ = oracle.group_bank(wl["q"], wl["k"], wl["w"], qbar, wbar, "bf16", 0, G, P, K,
                                        want_bank=True)
    n_checked = 0
    for g in range(T // G):
        a = g * G
        if a + 1 > P:
            assert np.array_equal(g_i[a], d_i[a])
            n_checked += 1
        else:
            assert (bank[g] == -1).all()
    assert n_checked > 10


def test_exact_recovery_and_bank_shape(oracle_lib):
    """Whenever a query's dense top-K lies in its candidate set C_i = bank U
    {t+1..i}, the bank result equals the dense result; otherwise it is a top-K of
    C_i.  Banks hold min(P, t+1) ascending prefix positions; the t+1 > P rule is
    strict; the trailing incomplete group uses the original indexer."""
    T, G, P, K = 203, 4, 48, 16
    wl = _gb(T=T, G=G, P=P, K=K, seed=11, H=3, Hs=2, d=8)
    q, k, w = _f64(wl["q"]), _f64(wl["k"]), _f64(wl["w"])
    qb, wb = _f64(wl["qbar"]), _f64(wl["wbar"])
    d_i, _ = oracle.prefill(wl["q"], wl["k"], wl["w"], "bf16", 0, K)
    g_i, g_s, bank, _ = oracle.group_bank(wl["q"], wl["k"], wl["w"], wl["qbar"], wl["wbar"], "bf16",
                                          0, G, P, K, want_bank=True)
    S = (w[:, :, None] * np.maximum(np.einsum("thc,sc->ths", q, k), 0)).sum(1)
    Sb = (wb[:, :, None] * np.maximum(np.einsum("ghc,sc->ghs", qb, k), 0)).sum(1)
    full_groups = T // G
    recovered = 0
    for i in range(T):
        g, t = i // G, i
        a = g * G
        if g >= full_groups or a + 1 <= P:
            assert np.array_equal(g_i[i], d_i[i]), i
            if g < len(bank):
                assert (bank[g] == -1).all()
            continue
        b = bank[g][bank[g] >= 0]
        assert len(b) == P and (np.diff(b) > 0).all() and b.max() <= a
        # the bank is a top-P of the group score over s <= a
        rb, _ = lexsort_topk(Sb[g:g + 1, :a + 1], np.ones((1, a + 1), bool), P)
        assert np.array_equal(b, rb[0])
        cand = np.concatenate([b, np.arange(a + 1, t + 1)])
        ri, rs = lexsort_topk(S[i:i + 1, cand], np.ones((1, len(cand)), bool), K)
        ref = np.full(K, -1, np.int32)
        sel = np.sort(cand[ri[0][ri[0] >= 0]])
        ref[:len(sel)] = sel
        assert np.array_equal(g_i[i], ref)
        dense = d_i[i][d_i[i] >= 0]
        if np.isin(dense, cand).all():
            assert np.array_equal(g_i[i], d_i[i])
            recovered += 1
    # with P = 3K and 3 heads some queries are fully covered
    assert recovered > 0


def test_eligibility_boundary(oracle_lib):
    """Anchor t with t+1 == P falls back; t+1 == P+1 builds a bank."""
    G, P = 4, 21
    wl = _gb(T=40, G=G, P=P, K=8, seed=12)
    _, _, bank, _ = oracle.group_bank(wl["q"], wl["k"], wl["w"], wl["qbar"], wl["wbar"], "bf16", 0,
                                      G, P, 8, want_bank=True)
    # anchors 0,4,...,36: anchor 20 sees exactly P = 21 keys and falls back;
    # anchor 24 sees 25 > 21 and builds a bank of P
    assert (bank[5] == -1).all() and (bank[6] >= 0).all()
    assert oracle.group_bank_pairs(40, 0, G, P) == _pairs_closed_form(40, 0, G, P)


def _pairs_closed_form(Tq, q_pos0, G, P):
    """Scored pairs: fallback queries score t+1 keys; a bank group scores its
    anchor prefix once, then each member r scores |bank| + r (Appendix A.2,
    Eq. (17) with |bank| = P)."""
    total = 0
    for g in range(-(-Tq // G)):
        a = q_pos0 + g * G
        members = min(G, Tq - g * G)
        if members == G and a + 1 > P:
            total += (a + 1) + G * P + G * (G - 1) // 2
        else:
            total += sum(a + r + 1 for r in range(members))
    return total


@pytest.mark.parametrize("Tq,q_pos0,G,P", [(203, 0, 4, 48), (160, 40, 16, 64), (65536, 0, 16, 8192),
                                           (131072, 0, 8, 4096)])
def test_pair_count_closed_form(oracle_lib, Tq, q_pos0, G, P):
    assert oracle.group_bank_pairs(Tq, q_pos0, G, P) == _pairs_closed_form(Tq, q_pos0, G, P)


def test_pair_count_matches_continuous_model(oracle_lib):
    """The discrete count approaches Eq. (19); config 5's count gives the 3.38 of
    Table 5(a) at G=16, P=8K, L=64K."""
    L, G, P = 65536, 16, 8192
    disc = oracle.group_bank_pairs(L, 0, G, P)
    base = L * (L + 1) // 2
    assert disc == 635_846_144 and base == 2_147_516_416
    assert round(base / disc, 2) == 3.38
    assert abs(disc / oracle.cost_prefill_reuse(L, G, P) - 1) < 1e-3


def test_group_bank_pairs_reported(oracle_lib):
    wl = _gb(T=120, G=4, P=30, K=8, seed=13)
    _, _, _, pairs = oracle.group_bank(wl["q"], wl["k"], wl["w"], wl["qbar"], wl["wbar"], "bf16", 0,
                                       4, 30, 8)
    assert pairs == _pairs_closed_form(120, 0, 4, 30)


# ----------------------------------------------------------- Table 5 pins

def _table5():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        panel, G, P, *vals = line.split()
        rows.append((panel, int(G), int(P[:-1]) * 1024, [float(v) for v in vals]))
    return rows


def test_table5_all_entries(oracle_lib):
    """All 108 printed speedups of Appendix A, Table 5 (a)-(c) from the cost
    model of Eq. (15)-(24) and (28)."""
    n = 0
    for panel, G, P, vals in _table5():
        for L, v in zip([16384, 32768, 65536, 131072], vals):
            if panel == "a":
                s = oracle.cost_prefill_base(L) / oracle.cost_prefill_reuse(L, G, P)
            elif panel == "b":
                s = oracle.cost_mtp_base_round(L) / oracle.cost_mtp_reuse_round(L, G, P)
            else:
                s = oracle.speedup_joint(L, G, P)
            assert math.isclose(round(s, 2), v), (panel, G, P, L, s, v)
            n += 1
    assert n == 108


# ------------------------------------------- training-free group query pins

def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_pool_mean_of_identical_rows_is_the_row(oracle_lib):
    """A group of G copies of one query pools to that query, bit for bit, and
    its gates to the same gates (catches a wrong 1/G scale or group stride)."""
    G, NG, H, d = 8, 5, 3, 16
    g = torch.Generator().manual_seed(21)
    base = to_bf16(torch.randn(NG, H, d, generator=g))
    wb = to_bf16(torch.rand(NG, H, generator=g)).float()  # 8-bit values: every sum is exact
    q = base.repeat_interleave(G, 0)
    w = wb.repeat_interleave(G, 0)
    qbar, wbar = oracle.pool_mean_bf16(q, w, G)
    assert np.array_equal(qbar, _bits(base))
    np.testing.assert_array_equal(wbar, wb.numpy())


@pytest.mark.parametrize("G", [4, 8, 16])
def test_pool_mean_exact_on_integers(oracle_lib, G):
    """Small integers: every sum is exact, so the pooled query is the exact mean
    (a library mean in fp64), which bf16 holds exactly; the trailing incomplete
    group, which never builds a bank, pools to zero."""
    wl = _gb(T=G * 7 + 3, G=G, P=16, K=8, seed=22 + G)
    q, w = wl["q"], wl["w"]
    qbar, wbar = oracle.pool_mean_bf16(q, w, G)
    full = (q.shape[0] // G) * G
    ref_q = _f64(q)[:full].reshape(-1, G, *q.shape[1:]).mean(1)
    ref_w = _f64(w)[:full].reshape(-1, G, w.shape[1]).mean(1)
    assert np.array_equal(qbar[:-1], _bits(to_bf16(torch.from_numpy(ref_q).float())))
    np.testing.assert_array_equal(wbar[:-1], ref_w.astype(np.float32))
    assert (qbar[-1] == 0).all() and (wbar[-1] == 0).all()
    assert np.abs(ref_q).max() > 0.2  # the case is not trivially zero


def _bf16_value(code):
    """The exact value of a bf16 bit pattern, as a Fraction."""
    from fractions import Fraction
    return Fraction(float(np.array([int(code) << 16], dtype=np.uint32).view(np.float32)[0]))


def _nearest_bf16(x):
    """The bf16 code nearest to the Fraction x, ties to the even code, found by
    comparing x exactly with the bf16 values around its float image."""
    f = np.float32(float(x))
    c = int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)
    best = None
    for cand in (c - 1, c, c + 1, c + 2, c ^ 0x8000):
        cand &= 0xFFFF
        if (cand & 0x7F80) == 0x7F80:  # inf / nan
            continue
        err = abs(_bf16_value(cand) - x)
        key = (err, cand & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_pool_mean_is_the_correctly_rounded_mean(oracle_lib):
    """Normal inputs: every pooled query element is the group's exact mean
    (rational arithmetic) rounded to the nearest bf16 with ties to even, and
    every pooled gate the exact mean rounded to the nearest fp32.  Group 0 is
    built so that its mean lies just above a bf16 midpoint by less than an
    fp32 sum of its members can resolve (members 2, 1 x 5, 1 + 2^-5, 2^-27 give
    1 + 2^-8 + 2^-30): a sum in fp32 would land on the midpoint and round to
    even (down); the correctly rounded mean rounds up.  Group 1 is an exact
    midpoint (1 + 2^-8), which rounds to even."""
    from fractions import Fraction
    G = 8
    wl = _gb(T=G * 12, G=G, P=16, K=8, seed=25, dist="normal", H=4, d=32)
    q, w = wl["q"].clone(), wl["w"].clone()
    q[0:G, 0, 0] = torch.tensor([2, 1, 1, 1, 1, 1, 1 + 2 ** -5, 2 ** -27], dtype=torch.float32).to(torch.bfloat16)
    q[G:2 * G, 0, 0] = torch.tensor([1, 1, 1, 1, 1, 1, 1, 1 + 2 ** -5], dtype=torch.float32).to(torch.bfloat16)
    qbar, wbar = oracle.pool_mean_bf16(q, w, G)
    assert qbar[0, 0, 0] == 0x3F81  # 1 + 2^-7: above the midpoint rounds up
    assert qbar[1, 0, 0] == 0x3F80  # 1 + 2^-8 exactly: the even neighbour, 1.0
    qb = _bits(q).reshape(-1, G, *q.shape[1:])
    qv = qb.astype(np.uint32) << 16
    qf = qv.view(np.float32)
    for g in range(qb.shape[0]):
        for e in np.ndindex(*qb.shape[2:]):
            x = sum(Fraction(float(qf[g, i][e])) for i in range(G)) / G
            assert qbar[g][e] == _nearest_bf16(x), (g, e)
    wg = w.numpy().reshape(-1, G, w.shape[1])
    for g in range(wg.shape[0]):
        for j in range(wg.shape[2]):
            x = sum(Fraction(float(v)) for v in wg[g, :, j]) / G
            lo = np.float32(float(x))  # the float nearest to x's float64 image
            cands = [np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))]
            errs = [abs(Fraction(float(c)) - x) for c in cands]
            m = min(errs)
            ok = [c for c, e in zip(cands, errs) if e == m]
            assert wbar[g, j] in ok, (g, j)

def test_pooled_bank_is_the_bank_of_the_mean(oracle_lib):
    """The pooling flag uses the pooled query as the group query with all H heads:
    on integer inputs (where a library mean is exact) it equals the bank built
    from the library-mean group query and gates."""
    T, G, P, K = 200, 8, 40, 12
    wl = _gb(T=T, G=G, P=P, K=K, seed=26)
    q, w = wl["q"], wl["w"]
    qb = torch.from_numpy(_f64(q).reshape(-1, G, *q.shape[1:]).mean(1)).float()
    wb = torch.from_numpy(_f64(w).reshape(-1, G, w.shape[1]).mean(1)).float()
    e_i, e_s, e_bank, e_pairs = oracle.group_bank(q, wl["k"], w, to_bf16(qb), wb, "bf16", 0, G, P, K,
                                                  want_bank=True)
    p_i, p_s, p_bank, p_pairs = oracle.group_bank(q, wl["k"], w, wl["qbar"], wl["wbar"], "bf16", 0,
                                                  G, P, K, flags=oracle.POOL_MEAN, want_bank=True)
    assert np.array_equal(e_i, p_i) and np.array_equal(e_s, p_s)
    assert np.array_equal(e_bank, p_bank) and e_pairs == p_pairs
    # and it is not the bank of the trained-query stand-in
    _, _, t_bank, _ = oracle.group_bank(q, wl["k"], w, wl["qbar"], wl["wbar"], "bf16", 0, G, P, K,
                                        want_bank=True)
    assert not np.array_equal(t_bank, p_bank)


def test_pooled_identical_group_recovers_dense(oracle_lib):
    """When every query of a group is the same, the pooled query is that query,
    so with K <= P every query's dense top-K lies in the bank (the exact
    recovery of Section 1) and the pooled result equals the dense one."""
    T, G, P, K = 160, 4, 32, 10
    wl = _gb(T=T, G=G, P=P, K=K, seed=27, dist="normal")
    q = wl["q"][::G].repeat_interleave(G, 0).contiguous()
    w = wl["w"][::G].repeat_interleave(G, 0).contiguous()
    d_i, d_s = oracle.prefill(q, wl["k"], w, "bf16", 0, K)
    p_i, p_s, bank, _ = oracle.group_bank(q, wl["k"], w, wl["qbar"], wl["wbar"], "bf16", 0, G, P, K,
                                          flags=oracle.POOL_MEAN, want_bank=True)
    assert (bank >= 0).any()
    # members r > 0 score the same as their anchor on the bank, plus the keys
    # after it; the dense top-K of the anchor's query over s <= t is inside
    # bank U (t_anchor, t] because a top-P over s <= t_anchor holds its top-K
    assert np.array_equal(d_i, p_i) and np.array_equal(d_s, p_s)


# ------------------------------------------------- MTP verification pins

def _e4m3_values(codes, scale):
    """E4M3 codes times their per-token scale, decoded by torch (fp64)."""
    return codes.view(torch.float8_e4m3fn).double() * scale.double()[..., None]


def _mtp_dense_ref(q, kv, w, N, m, K):
    """Original indexer for a window's queries: query r sees keys 0..N-1+r."""
    S = (w[:, :, None] * np.maximum(np.einsum("rhc,sc->rhs", q, kv), 0)).sum(1)
    valid = np.arange(kv.shape[0])[None, :] <= (N - 1 + np.arange(m))[:, None]
    return lexsort_topk(S, valid, K)


def test_mtp_pairs_are_eq20_21(oracle_lib):
    """The discrete count of an MTP round is Eq. (20)-(21): m N + m(m-1)/2 when
    the window falls back (N <= P), else (m/G) N + m P + (m/2)(m/G + G - 2)."""
    m, P = 16, 2048
    for G in (4, 8, 16):
        for N in (1, 700, P - 1, P, P + 1, 3 * P + 5, 131072):
            want = m * N + m * (m - 1) // 2 if N <= P else (m // G) * N + m * P + (m // 2) * (m // G + G - 2)
            assert oracle.mtp_pairs([N], m, G, P) == want, (G, N)
    assert oracle.mtp_pairs([100, 5000], m, 4, P) == sum(oracle.mtp_pairs([n], m, 4, P) for n in (100, 5000))


def test_mtp_eligible_window_is_the_group_bank(oracle_lib):
    """N > P: every group of the window reuses a bank, exactly as prefill
    grouping does for groups starting at query N-1 (anchor g sees N + gG keys)."""
    m, G, P, K, N = 16, 4, 40, 12, 150
    wl = make_mtp(B=1, N=N + m - 1, m=m, H=3, Hs=2, d=16, topk=K, G=G, P=P, dist="int", seed=30,
                  prefix_lens=[N])
    t = wl.tensors
    mi, ms, mb, pairs = oracle.mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], t["qbar"], t["wbar"],
                                   t["prefix_lens"], G, P, K, want_bank=True)
    kv = to_bf16(_e4m3_values(t["k_cache"][0], t["k_scale"][0]).float())  # exact: small integers
    gi, gs, gb, gp = oracle.group_bank(t["q"][0], kv, t["w"][0], t["qbar"][0], t["wbar"][0], "bf16", N - 1, G, P,
                                       K, want_bank=True)
    assert np.array_equal(mi, gi) and np.array_equal(ms, gs)
    assert np.array_equal(mb[0], gb) and (mb >= 0).all() and pairs == gp


def test_mtp_window_falls_back_as_a_whole(oracle_lib):
    """N <= P: the whole window uses the original indexer even though its later
    anchors see more than P keys (prefill grouping would build their banks)."""
    m, G, P, K, N = 16, 4, 40, 12, 33  # anchors see 33, 37, 41, 45 keys
    wl = make_mtp(B=1, N=N + m - 1, m=m, H=3, Hs=2, d=16, topk=K, G=G, P=P, dist="int", seed=31,
                  prefix_lens=[N])
    t = wl.tensors
    mi, ms, mb, pairs = oracle.mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], t["qbar"], t["wbar"],
                                   t["prefix_lens"], G, P, K, want_bank=True)
    assert (mb == -1).all() and pairs == m * N + m * (m - 1) // 2
    kv = _e4m3_values(t["k_cache"][0], t["k_scale"][0]).numpy()
    ri, rs = _mtp_dense_ref(_f64(t["q"][0]), kv, _f64(t["w"][0]), N, m, K)
    assert np.array_equal(mi, ri)
    np.testing.assert_allclose(ms, rs, rtol=1e-12)
    kvb = to_bf16(torch.from_numpy(kv).float())
    _, _, gb, _ = oracle.group_bank(t["q"][0], kvb, t["w"][0], t["qbar"][0], t["wbar"][0], "bf16", N - 1, G, P, K,
                                    want_bank=True)
    assert (gb[2:] >= 0).any()  # the per-group rule would differ here


def test_mtp_brute_force_batch(oracle_lib):
    """A batch mixing fallback and bank windows against a direct restatement
    of the rule in numpy (bank = top-P of the group score over the anchor's
    visible keys; members rank bank plus post-anchor keys), scales included."""
    B, m, G, P, K, H, Hs, d = 3, 16, 8, 24, 10, 3, 2, 8
    lens = [20, 24, 25]
    wl = make_mtp(B=B, N=60, m=m, H=H, Hs=Hs, d=d, topk=K, G=G, P=P, dist="normal", seed=32,
                  prefix_lens=lens)
    t = wl.tensors
    mi, ms, mb, _ = oracle.mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], t["qbar"], t["wbar"],
                               t["prefix_lens"], G, P, K, want_bank=True)
    for b, N in enumerate(lens):
        kv = _e4m3_values(t["k_cache"][b], t["k_scale"][b]).numpy()
        q, w = _f64(t["q"][b]), _f64(t["w"][b])
        S = (w[:, :, None] * np.maximum(np.einsum("rhc,sc->rhs", q, kv), 0)).sum(1)
        if N <= P:
            ri, _ = _mtp_dense_ref(q, kv, w, N, m, K)
            assert np.array_equal(mi[b * m:(b + 1) * m], ri) and (mb[b] == -1).all()
            continue
        qb, wb = _f64(t["qbar"][b]), _f64(t["wbar"][b])
        Sb = (wb[:, :, None] * np.maximum(np.einsum("ghc,sc->ghs", qb, kv), 0)).sum(1)
        for g in range(m // G):
            a = N - 1 + g * G
            bank, _ = lexsort_topk(Sb[g:g + 1, :a + 1], np.ones((1, a + 1), bool), P)
            assert np.array_equal(mb[b, g], bank[0])
            for i in range(G):
                r = g * G + i
                cand = np.concatenate([bank[0], np.arange(a + 1, a + 1 + i)])
                ci, _ = lexsort_topk(S[r:r + 1, cand], np.ones((1, len(cand)), bool), K)
                assert np.array_equal(mi[b * m + r], np.sort(cand[ci[0]])), (b, r)


def test_mtp_rows_and_pooling(oracle_lib):
    """Requested rows (any order) equal the full result's rows; mean pooling
    equals passing the pooled query explicitly."""
    B, m, G, P, K = 2, 16, 4, 30, 8
    wl = make_mtp(B=B, N=90, m=m, H=4, Hs=4, d=16, topk=K, G=G, P=P, dist="int", seed=33, prefix_lens=[70, 31])
    t = wl.tensors
    fi, fs, fb, _ = oracle.mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], t["qbar"], t["wbar"],
                               t["prefix_lens"], G, P, K, want_bank=True)
    rows = [17, 3, 30, 0, 31]
    ri, rs, _, _ = oracle.mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], t["qbar"], t["wbar"],
                              t["prefix_lens"], G, P, K, rows=rows)
    assert np.array_equal(ri, fi[rows]) and np.array_equal(rs, fs[rows])
    pq = np.stack([oracle.pool_mean_bf16(t["q"][b], t["w"][b], G)[0] for b in range(B)])
    pw = np.stack([oracle.pool_mean_bf16(t["q"][b], t["w"][b], G)[1] for b in range(B)])
    ei, _, eb, _ = oracle.mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], pq, pw, t["prefix_lens"], G, P, K,
                              want_bank=True)
    pi, _, pb, _ = oracle.mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], None, None, t["prefix_lens"], G, P, K,
                              flags=oracle.POOL_MEAN, want_bank=True)
    assert np.array_equal(ei, pi) and np.array_equal(eb, pb) and not np.array_equal(eb, fb)


def test_mtp_no_bank_is_the_original_indexer(oracle_lib):
    """NO_BANK: every window, eligible or not, ranks each query's visible keys."""
    m, G, P, K = 16, 4, 30, 9
    lens = [50, 10]
    wl = make_mtp(B=2, N=80, m=m, H=3, Hs=2, d=16, topk=K, G=G, P=P, dist="normal", seed=34, prefix_lens=lens)
    t = wl.tensors
    mi, ms, mb, pairs = oracle.mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], t["qbar"], t["wbar"],
                                   t["prefix_lens"], G, P, K, flags=oracle.NO_BANK, want_bank=True)
    assert (mb == -1).all() and pairs == sum(m * N + m * (m - 1) // 2 for N in lens)
    for b, N in enumerate(lens):
        kv = _e4m3_values(t["k_cache"][b], t["k_scale"][b]).numpy()
        ri, rs = _mtp_dense_ref(_f64(t["q"][b]), kv, _f64(t["w"][b]), N, m, K)
        assert np.array_equal(mi[b * m:(b + 1) * m], ri)
        np.testing.assert_allclose(ms[b * m:(b + 1) * m], rs, rtol=1e-12)


# ------------------------------------------------- calibration pins

LAYERS = __file__.replace("test_oracle_pins.py", "golden/layer_configs.txt")


def _table5c_128k():
    """Printed joint speedups at 128K, Table 5(c): {(G, P): value}."""
    return {(G, P): v[3] for panel, G, P, v in _table5() if panel == "c"}


def _layer_tables():
    tabs = {}
    for line in open(LAYERS):
        if line.startswith("#") or not line.strip():
            continue
        t, model, stat, G, P, cnt, layers = line.split()
        ls = []
        for part in layers.split(","):
            lo, _, hi = part.partition("-")
            ls += list(range(int(lo), int(hi or lo) + 1))
        assert len(ls) == int(cnt), (t, G, P)
        tabs.setdefault((int(t), model, stat), {}).update({layer: (int(G), int(P[:-1]) * 1024) for layer in ls})
    return tabs


def test_union_sizes_closed_forms(oracle_lib):
    """Identical rows unite to K, disjoint rows to G*K, empty slots count for
    nothing, a trailing incomplete group has no anchor; random rows against
    Python set unions."""
    import oracle.calib as calib
    K, G = 6, 4
    same = np.tile(np.arange(10, 10 + K), (G, 1))
    disjoint = np.arange(G * K).reshape(G, K)
    padded = np.array([[1, 2, 3, -1, -1, -1], [2, 3, 4, 5, -1, -1], [-1] * 6, [9, -1, -1, -1, -1, -1]])
    idx = np.concatenate([same, disjoint, padded, same[:2]])
    assert list(calib.union_sizes(idx, G)) == [K, G * K, 6]
    rng = np.random.default_rng(3)
    r = np.sort(rng.choice(50, size=(16, 8), replace=True), axis=1)
    want = [len(set(r[g * 8:(g + 1) * 8].ravel().tolist())) for g in range(2)]
    assert list(calib.union_sizes(r, 8)) == want


def test_union_stats_and_overlap(oracle_lib):
    import oracle.calib as calib
    assert calib.union_stat(range(1, 11), "p90") == 9
    assert calib.union_stat(range(1, 21), "p90") == 18
    assert calib.union_stat([7], "p90") == 7
    assert calib.union_stat([1, 2, 9], "max") == 9 and calib.union_stat([1, 2, 9], "mean") == 4
    a = np.array([[1, 4, 7, -1], [0, 1, 2, 3]])
    b = np.array([[4, 5, 7, 9], [-1, -1, -1, -1]])
    assert list(calib.overlap_counts(a, b)) == [2, 0]


def test_setting_selection_follows_table5(oracle_lib):
    """Eq. (5) picks the largest printed 128K joint speedup of Table 5(c) among
    the settings whose P covers the union statistic of their G."""
    import oracle.calib as calib
    s = _table5c_128k()
    for stats in ({4: 100, 8: 100, 16: 100}, {4: 5000, 8: 9000, 16: 20000}, {4: 4096, 8: 8193, 16: 16385},
                  {4: 30000, 8: 30000, 16: 30000}):
        feasible = {k: v for k, v in s.items() if stats[k[0]] <= k[1]}
        got = calib.select_setting(stats)
        if not feasible:
            assert got is None
            continue
        best = max(feasible.values())
        assert s[got] == best, (stats, got, best)


def test_layerwise_speedup_eq27(oracle_lib):
    """A uniform assignment gives that setting's Table 5(c) value; a mixed one
    sums scoring counts over layers (Eq. (27)), so it lies between its settings'
    values and equals |layers| over the sum of reciprocal speedups; the printed
    layer tables partition the 61 (DeepSeek-V3.2) and 78 (GLM-5.1) layers."""
    import oracle.calib as calib
    s = _table5c_128k()
    for (G, P), v in s.items():
        assert round(calib.layerwise_speedup([(G, P)] * 5, 131072), 2) == v
    tabs = _layer_tables()
    assert {k[1]: len(v) for k, v in tabs.items()} == {"deepseek-v3.2": 61, "glm-5.1": 78}
    for key, layers in tabs.items():
        assert sorted(layers) == list(range(len(layers))), key
        settings = [layers[i] for i in range(len(layers))]
        sp = calib.layerwise_speedup(settings, 131072)
        vals = [s[x] for x in settings]
        assert min(vals) - 0.01 <= sp <= max(vals) + 0.01
        # counts add: base / speedup is each layer's reuse count (base is shared)
        harm = len(vals) / sum(1.0 / v for v in vals)
        assert abs(sp / harm - 1) < 0.01, (key, sp, harm)


# ------------------------------------------- group query construction pins

def _gq_inputs(Tq=48, dc=32, dh=40, Hs=4, d=16, seed=40):
    g = torch.Generator().manual_seed(seed)
    c = torch.randn(Tq, dc, generator=g).to(torch.bfloat16)
    h = torch.randn(Tq, dh, generator=g).to(torch.bfloat16)
    wq = (torch.randn(Hs * d, dc, generator=g) / dc ** 0.5).to(torch.bfloat16)
    wg = (torch.randn(Hs, dh, generator=g) / dh ** 0.5).to(torch.bfloat16)
    return c, h, wq, wg


def test_group_query_mean_pooling_init(oracle_lib):
    """W_pool = [0, 0, I] (the initialisation of Appendix C.3) makes cbar the
    group mean; with no rotary part, qbar is W_Q times that mean and the gates
    are the sigmoid of W_G times the mean hidden state."""
    from oracle import group_query as gq
    c, h, wq, wg = _gq_inputs()
    dc, G, Hs, d = 32, 8, 4, 16
    wp = np.concatenate([np.zeros((dc, 2 * dc)), np.eye(dc)], 1)
    q, w = gq.group_query(c, h, wp, wq, wg, G, Hs, d, rope_dim=0)
    cm = _bf16(c.double().reshape(6, G, dc).mean(1)).double().numpy()          # bf16 operand, twice
    want = (cm @ wq.double().numpy().T).reshape(6, Hs, d)
    np.testing.assert_allclose(q, _bf16(want).double().numpy(), rtol=0, atol=0)
    hm = _bf16(h.double().reshape(6, G, -1).mean(1)).double().numpy()
    np.testing.assert_allclose(w, 1 / (1 + np.exp(-(hm @ wg.double().numpy().T))), rtol=1e-12)


def test_group_query_pool_order_and_single_row(oracle_lib):
    """The three pooled blocks are max, min, mean in that order; a group of one
    row pools to the row three times."""
    from oracle import group_query as gq
    c = torch.tensor([[1.0, -2.0], [3.0, 5.0], [-1.0, 0.5], [0.0, 0.0]])
    pc, ph = gq.pool(c, c, 2)
    assert np.array_equal(pc, [[3, 5, 1, -2, 2, 1.5], [0, 0.5, -1, 0, -0.5, 0.25]])
    pc1, _ = gq.pool(c, c, 1)
    assert np.array_equal(pc1[:, :2], pc1[:, 2:4]) and np.array_equal(pc1[:, 2:4], pc1[:, 4:])


def test_group_query_rope(oracle_lib):
    """Rotary embedding: identity at position 0 and past rope_dim; each pair
    keeps its length; the pair (0, rope_dim/2) turns by the anchor position
    itself (frequency 1) and the two heads of a group turn alike."""
    from oracle import group_query as gq
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 2, 16))
    pos = np.array([0, 5, 40])
    y = gq.rope(x, pos, 8, 10000.0)
    assert np.array_equal(y[0], x[0]) and np.array_equal(y[:, :, 8:], x[:, :, 8:])
    for i in range(4):
        np.testing.assert_allclose(np.hypot(y[..., i], y[..., i + 4]), np.hypot(x[..., i], x[..., i + 4]))
    a, b = x[2, 1, 0], x[2, 1, 4]
    np.testing.assert_allclose([y[2, 1, 0], y[2, 1, 4]], [a * math.cos(40) - b * math.sin(40),
                                                          b * math.cos(40) + a * math.sin(40)])


def test_group_query_anchor_positions_and_tail(oracle_lib):
    """Group g's query is rotated at q_pos0 + gG (shifting q_pos0 by G shifts
    the result by one group); an incomplete last group gets zeros."""
    from oracle import group_query as gq
    c, h, wq, wg = _gq_inputs(Tq=52)
    rng = np.random.default_rng(4)
    wp = rng.standard_normal((32, 96)) / 10
    q0, w0 = gq.group_query(c, h, wp, wq, wg, 8, 4, 16, q_pos0=16, rope_dim=8)
    q1, _ = gq.group_query(c[8:], h[8:], wp, wq, wg, 8, 4, 16, q_pos0=24, rope_dim=8)
    np.testing.assert_allclose(q0[1:6], q1[:5])
    assert q0.shape == (7, 4, 16) and (q0[6] == 0).all() and (w0[6] == 0).all()
    # a different anchor position changes the rotated part only
    q2, _ = gq.group_query(c, h, wp, wq, wg, 8, 4, 16, q_pos0=17, rope_dim=8)
    assert np.array_equal(q0[:6, :, 8:], q2[:6, :, 8:]) and not np.array_equal(q0[:6, :, :8], q2[:6, :, :8])
