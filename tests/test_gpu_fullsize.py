"""GPU parity at the full workload sizes, in the launch configuration bench.py
times, on sampled rows the oracle computes one by one: the 16K bf16 prefill,
the 128K fp8 prefill in 4096-query chunks, the 32 x 256K decode and the 64K
ADIndex bank with G=16, P=8192.  Random inputs follow the tolerance rule;
integer-valued inputs at the same shapes must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import compare
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsa_amd as m
    m.lib()
    return m


def _sample(T, n, seed, always=()):
    rng = np.random.default_rng(seed)
    r = np.concatenate([rng.choice(T, n, replace=False), np.asarray(always, np.int64)])
    return np.unique(r[(r >= 0) & (r < T)])


def _host(t):
    return {k: v.cpu() for k, v in t.items()}


def _prefill_rows(wl_h, dt, rows, K):
    return oracle.prefill(wl_h["q"], wl_h["k"], wl_h["w"], dt, 0, K, wl_h.get("q_scale"), wl_h.get("k_scale"),
                          rows=rows)


def _score_of(wl_h, dt, rows):
    def f(r, keys):
        return oracle.score_pairs(wl_h["q"], wl_h["k"], wl_h["w"], np.full(len(keys), rows[r]), keys, dt, dt,
                                  wl_h.get("q_scale"), wl_h.get("k_scale"))
    return f


@pytest.mark.parametrize("dist", ["normal", "int"])
def test_dsa_prefill_16k_bf16(dsa, dist):
    """T=16384, H=64, d=128, top-2048, bf16, one call."""
    wl = make_workload(2, seed=3, device="cuda", dist=dist)
    t = wl.tensors
    gi, gs = dsa.indexer_prefill(t["q"], t["k"], t["w"], 0, 2048)
    torch.cuda.synchronize()
    rows = _sample(16384, 20, 3, always=(0, 1, 2046, 2047, 2048, 16383))
    h = _host(t)
    ri, rs = _prefill_rows(h, "bf16", rows, 2048)
    compare(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, dist == "int", _score_of(h, "bf16", rows))


@pytest.mark.parametrize("dist", ["normal", "int"])
def test_long_prefill_128k_fp8_chunked(dsa, dist):
    """T=131072, fp8 with per-token scales, 32 causal query chunks of 4096
    (the bench.py launch configuration); the score matrix is never stored."""
    T, K, C = 131072, 2048, 4096
    wl = make_workload(3, seed=4, device="cuda", dist=dist)
    t = wl.tensors
    out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    osc = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(dsa.workspace_prefill(C, T, 64, 128, K, dsa.DSAIDX_FP8_E4M3), dtype=torch.uint8,
                     device="cuda")
    for c in range(T // C):
        q0, q1 = c * C, (c + 1) * C
        dsa.indexer_prefill(t["q"][q0:q1], t["k"][:q1], t["w"][q0:q1], q0, K, t["q_scale"][q0:q1],
                            t["k_scale"][:q1], out_idx=out[q0:q1], out_score=osc[q0:q1], ws=ws)
    torch.cuda.synchronize()
    rows = _sample(T, 12, 4, always=(0, 2047, 4095, 4096, 65535, T - 1))
    h = _host(t)
    ri, rs = _prefill_rows(h, "fp8", rows, K)
    compare(out.cpu().numpy()[rows], osc.cpu().numpy()[rows], ri, rs, dist == "int", _score_of(h, "fp8", rows))


@pytest.mark.parametrize("dist", ["normal", "int"])
def test_decode_256k(dsa, dist):
    """32 sequences x 262144 cached E4M3 keys, bf16 queries, top-2048."""
    B, N, K = 32, 262144, 2048
    wl = make_workload(4, seed=5, device="cuda", dist=dist)
    t = wl.tensors
    gi, gs = dsa.indexer_decode(t["q"], t["k_cache"], t["k_scale"], t["w"], t["seq_lens"], K)
    torch.cuda.synchronize()
    rows = np.array([0, 13, 31])
    h = _host(t)
    ri, rs = oracle.decode(h["q"], h["k_cache"], h["k_scale"], h["w"], h["seq_lens"], K, rows=rows)
    kc = h["k_cache"].reshape(B * N, -1)
    ks = h["k_scale"].reshape(B * N)

    def score_of(r, keys):
        return oracle.score_pairs(h["q"], kc, h["w"], np.full(len(keys), rows[r]), rows[r] * N + keys, "bf16",
                                  "fp8", None, ks)
    compare(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, dist == "int", score_of)


def test_adindex_256k_bank(dsa):
    """The pages' length, T=262144 (G=16, P=8192, 64-head group indexer,
    integer inputs): the banks and refined rows of sampled groups match the
    oracle exactly, early, in the middle and at the end of the sequence."""
    T, G, P, K = 262144, 16, 8192, 2048
    wl = make_workload(5, seed=7, device="cuda", dist="int", T=T)
    t = wl.tensors
    gi, gs, gb = dsa.indexer_group_bank(t["q"], t["k"], t["w"], t["qbar"], t["wbar"], 0, G, P, K, want_bank=True)
    torch.cuda.synchronize()
    rows = np.array([8224, 131077, 262143])
    h = _host(t)
    ri, rs, rb, pairs = oracle.group_bank(h["q"], h["k"], h["w"], h["qbar"], h["wbar"], "bf16", 0, G, P, K,
                                          rows=rows, want_bank=True)
    assert pairs == dsa.indexer_group_bank_pairs(T, 0, G, P)
    gbank = gb.cpu().numpy()
    for g in np.unique(rows // G):
        assert np.array_equal(gbank[g], rb[g])
    compare(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, True)


@pytest.mark.parametrize("pool", [False, True])
@pytest.mark.parametrize("dist", ["normal", "int"])
def test_adindex_64k_bank(dsa, dist, pool):
    """T=65536, G=16, P=8192, 64-head group indexer (or, with pooling, the
    training-free mean-pooled group query); sampled rows in the fallback groups
    (anchor+1 <= P) and in bank groups, with their banks."""
    T, G, P, K = 65536, 16, 8192, 2048
    flags = dsa.POOL_MEAN if pool else 0
    wl = make_workload(5, seed=6, device="cuda", dist=dist)
    t = wl.tensors
    gi, gs, gb = dsa.indexer_group_bank(t["q"], t["k"], t["w"], None if pool else t["qbar"],
                                        None if pool else t["wbar"], 0, G, P, K, flags=flags, want_bank=True)
    torch.cuda.synchronize()
    rows = np.unique(np.array([5, 8191, 8192, 8193, 8207, 20000, 33333, 50001, 65520, 65535]))
    h = _host(t)
    ri, rs, rb, pairs = oracle.group_bank(h["q"], h["k"], h["w"], h["qbar"], h["wbar"], "bf16", 0, G, P, K,
                                          flags=flags, rows=rows, want_bank=True)
    if pool:  # score the banks with the oracle's pooled query
        pq, pw = oracle.pool_mean_bf16(h["q"], h["w"], G)
        h["qbar"] = torch.from_numpy(pq.view(np.int16)).view(torch.bfloat16)
        h["wbar"] = torch.from_numpy(pw)
    assert pairs == dsa.indexer_group_bank_pairs(T, 0, G, P) == 635_846_144
    gbank = gb.cpu().numpy()
    groups = np.unique(rows // G)
    # banks of the sampled groups: the oracle's bank is a top-P of the group score
    for g in groups:
        if g * G + 1 <= P:
            assert (gbank[g] == -1).all() and (rb[g] == -1).all()
            continue
        v = rb[g][rb[g] >= 0]
        bs = oracle.score_pairs(h["qbar"], h["k"], h["wbar"], np.full(len(v), g), v, "bf16", "bf16")[None, :]

        def bank_score(r, keys, g=g):
            return oracle.score_pairs(h["qbar"], h["k"], h["wbar"], np.full(len(keys), g), keys, "bf16", "bf16")
        compare(gbank[g:g + 1], None, rb[g:g + 1], bs, dist == "int", bank_score, label=f"bank {g}")
    if dist == "int":
        compare(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, True)
    else:
        # rows whose group bank equals the oracle's bank are compared under the
        # tolerance rule (the banks themselves were checked above)
        same = [np.array_equal(rb[r // G], gbank[r // G]) for r in rows]
        sel = np.nonzero(same)[0]
        assert len(sel) >= len(rows) // 2
        compare(gi.cpu().numpy()[rows][sel], gs.cpu().numpy()[rows][sel], ri[sel], rs[sel], False,
                lambda r, keys: _score_of(h, "bf16", rows)(sel[r], keys))


@pytest.mark.parametrize("G,P", [(8, 8192), (16, 16384)])
def test_mtp_256k_windows(dsa, G, P):
    """MTP verification at 256K: 4 sequences of 262144 E4M3 keys, 16-query
    windows (one ending at the cache end, one shorter, one at the P boundary),
    an 8-head group indexer; sampled rows and their banks against the oracle."""
    from workloads import make_mtp
    B, N, m, K = 4, 262144, 16, 2048
    lens = [N - m + 1, 100000, P, P + 1]
    wl = make_mtp(B=B, N=N, m=m, H=64, Hs=8, d=128, topk=K, G=G, P=P, dist="int", seed=60 + G, device="cuda",
                  prefix_lens=lens)
    t = wl.tensors
    gi, gs, gb = dsa.indexer_mtp(t["q"], t["k_cache"], t["k_scale"], t["w"], t["qbar"], t["wbar"],
                                 t["prefix_lens"], G, P, K, want_bank=True)
    torch.cuda.synchronize()
    rows = np.array([0, 7, 15, 16, 25, 40, 47, 48, 60, 63])
    h = _host(t)
    ri, rs, rb, _ = oracle.mtp(h["q"], h["k_cache"], h["k_scale"], h["w"], h["qbar"], h["wbar"], h["prefix_lens"],
                               G, P, K, rows=rows, want_bank=True)
    gb = gb.cpu().numpy()
    for r in rows:  # the banks of the sampled rows' groups (window 2 falls back: all -1)
        b, g = r // m, (r % m) // G
        assert np.array_equal(gb[b, g], rb[b, g]), (b, g)
    assert (gb[2] == -1).all() and (gb[3] >= 0).all()
    compare(gi.reshape(B * m, K).cpu().numpy()[rows], gs.reshape(B * m, K).cpu().numpy()[rows], ri, rs, True)
