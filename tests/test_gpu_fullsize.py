"""GPU parity at the full workload sizes, in the launch configuration bench.py
times: every row of the 16K bf16 prefill and of the 32 x 256K decode, and at
least 512 stratified rows (always the last 16) of the 128K fp8 prefill in
4096-query chunks and of the 64K ADIndex bank with G=16, P=8192, whose sample
also covers the groups around the fallback/bank boundary.  The bank path is
also checked at the other budgets of the pages' (G, P) grid, P = 4096 and
16384 with G = 4, 8, 16, and with E4M3 inputs at 20K tokens.  Random inputs
follow the tolerance rule; integer-valued inputs at the same shapes must
match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import compare, pair_refs, refine_over_bank
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


def _stratified(T, n, always=()):
    """n rows evenly spread over 0..T-1, the last 16 rows and `always`."""
    r = np.concatenate([np.linspace(0, T - 1, n).astype(np.int64), np.arange(T - 16, T),
                        np.asarray(always, np.int64)])
    return np.unique(r[(r >= 0) & (r < T)])


def _host(t):
    return {k: v.cpu() for k, v in t.items()}


def _prefill_rows(wl_h, dt, rows, K):
    return oracle.prefill(wl_h["q"], wl_h["k"], wl_h["w"], dt, 0, K, wl_h.get("q_scale"), wl_h.get("k_scale"),
                          rows=rows)


def _refs(wl_h, dt, rows):
    """(score_of, cond_of) of the oracle for the given query rows."""
    return pair_refs(wl_h["q"], wl_h["k"], wl_h["w"], rows, dt, dt, wl_h.get("q_scale"), wl_h.get("k_scale"))


def _cmp(gi, gs, ri, rs, exact, refs, sel=None, label=""):
    score_of, cond_of = refs
    if sel is None:
        compare(gi, gs, ri, rs, exact, score_of, label=label, ref_cond_of=cond_of)
    else:
        compare(gi, gs, ri, rs, exact, lambda r, keys: score_of(sel[r], keys), label=label,
                ref_cond_of=lambda r, keys: cond_of(sel[r], keys))


@pytest.mark.parametrize("dist", ["normal", "int"])
def test_dsa_prefill_16k_bf16(dsa, dist):
    """T=16384, H=64, d=128, top-2048, bf16, one call: every row, with scores."""
    wl = make_workload(2, seed=3, device="cuda", dist=dist)
    t = wl.tensors
    gi, gs = dsa.indexer_prefill(t["q"], t["k"], t["w"], 0, 2048)
    torch.cuda.synchronize()
    rows = np.arange(16384)
    h = _host(t)
    ri, rs = _prefill_rows(h, "bf16", rows, 2048)
    _cmp(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, dist == "int", _refs(h, "bf16", rows))


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
    rows = _stratified(T, 512, always=(0, 2047, 4095, 4096, 6143, 6144, 65535))
    h = _host(t)
    ri, rs = _prefill_rows(h, "fp8", rows, K)
    _cmp(out.cpu().numpy()[rows], osc.cpu().numpy()[rows], ri, rs, dist == "int", _refs(h, "fp8", rows))


@pytest.mark.parametrize("dist", ["normal", "int"])
def test_decode_256k(dsa, dist):
    """32 sequences x 262144 cached E4M3 keys, bf16 queries, top-2048: every
    row, with scores."""
    B, N, K = 32, 262144, 2048
    wl = make_workload(4, seed=5, device="cuda", dist=dist)
    t = wl.tensors
    gi, gs = dsa.indexer_decode(t["q"], t["k_cache"], t["k_scale"], t["w"], t["seq_lens"], K)
    torch.cuda.synchronize()
    rows = np.arange(B)
    h = _host(t)
    ri, rs = oracle.decode(h["q"], h["k_cache"], h["k_scale"], h["w"], h["seq_lens"], K, rows=rows)
    kc = h["k_cache"].reshape(B * N, -1)
    ks = h["k_scale"].reshape(B * N)

    refs = pair_refs(h["q"], kc, h["w"], rows, "bf16", "fp8", None, ks, key_of=lambda r, keys: rows[r] * N + keys)
    _cmp(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, dist == "int", refs)


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
    training-free mean-pooled group query); 512 stratified rows, the last 16
    and the groups on both sides of the fallback/bank boundary (the last
    fallback group ends at row 8191; group 512 is the first bank group), with
    their banks."""
    T, G, P, K = 65536, 16, 8192, 2048
    flags = dsa.POOL_MEAN if pool else 0
    wl = make_workload(5, seed=6, device="cuda", dist=dist)
    t = wl.tensors
    gi, gs, gb = dsa.indexer_group_bank(t["q"], t["k"], t["w"], None if pool else t["qbar"],
                                        None if pool else t["wbar"], 0, G, P, K, flags=flags, want_bank=True)
    torch.cuda.synchronize()
    rows = _stratified(T, 512, always=np.concatenate([[5], np.arange(8160, 8240)]))
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
        brefs = pair_refs(h["qbar"], h["k"], h["wbar"], [g], "bf16", "bf16")
        _cmp(gbank[g:g + 1], None, rb[g:g + 1], brefs[0](0, v)[None, :], dist == "int", brefs, label=f"bank {g}")
    if dist == "int":
        compare(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, True)
    else:
        # rows whose group bank equals the oracle's bank are compared with the
        # oracle's rows under the tolerance rule (the banks themselves were
        # checked above); a bank that differs only by tolerated swaps is a
        # valid bank too, and the rows of its group must then be the top K of
        # Eq. (14) over that bank, scored by the oracle
        same = np.array([np.array_equal(rb[r // G], gbank[r // G]) for r in rows])
        sel = np.nonzero(same)[0]
        _cmp(gi.cpu().numpy()[rows][sel], gs.cpu().numpy()[rows][sel], ri[sel], rs[sel], False,
             _refs(h, "bf16", rows), sel=sel)
        other = rows[~same]
        if len(other):
            oi, osc = refine_over_bank(h, gbank, other, G, K)
            _cmp(gi.cpu().numpy()[other], gs.cpu().numpy()[other], oi, osc, False, _refs(h, "bf16", other),
                 label="own bank")


@pytest.mark.parametrize("P", [4096, 16384])
@pytest.mark.parametrize("G", [4, 8, 16])
def test_group_bank_budgets(dsa, G, P):
    """The bank path at the budgets of the pages' (G, P) grid that the 64K
    workload does not use (P = 4096 and 16384; Eq. (5) searches G in {4, 8, 16}
    and P in {4K, 8K, 16K}): 64 heads, d = 128, bf16 integer inputs over
    P + 6144 tokens, so fallback groups, the boundary and bank groups all
    occur; banks and rows of sampled groups match the oracle bit for bit.
    G = 4 refines in the general kernel, G = 8 and 16 in the dense kernel's
    gather mode."""
    T, K = P + 6144, 2048
    wl = make_workload(5, seed=80 + G, device="cuda", dist="int", T=T, G=G, P=P)
    t = wl.tensors
    gi, gs, gb = dsa.indexer_group_bank(t["q"], t["k"], t["w"], t["qbar"], t["wbar"], 0, G, P, K, want_bank=True)
    torch.cuda.synchronize()
    b0 = -(-P // G) * G  # first row of the first bank group
    rows = _stratified(T, 48, always=np.concatenate([np.arange(b0 - G, b0 + G + 1), [P - 1, P]]))
    h = _host(t)
    ri, rs, rb, pairs = oracle.group_bank(h["q"], h["k"], h["w"], h["qbar"], h["wbar"], "bf16", 0, G, P, K,
                                          rows=rows, want_bank=True)
    assert pairs == dsa.indexer_group_bank_pairs(T, 0, G, P)
    gbank = gb.cpu().numpy()
    for g in np.unique(rows // G):
        assert np.array_equal(gbank[g], rb[g]), g
    compare(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, True)


@pytest.mark.parametrize("dist", ["int", "normal"])
def test_group_bank_fp8_20k(dsa, dist):
    """E4M3 q, k and group query with per-token scales at T = 20480 (G = 16,
    P = 8192): banks and sampled rows match the oracle (bit for bit on
    integer inputs, under the tolerance rule on normal ones, where a row
    whose bank differs by tolerated swaps is checked against Eq. (14) over
    the GPU's bank)."""
    T, G, P, K = 20480, 16, 8192, 2048
    wl = make_workload(5, seed=90, device="cuda", dist=dist, T=T, dtype="fp8")
    t = wl.tensors
    gi, gs, gb = dsa.indexer_group_bank(t["q"], t["k"], t["w"], t["qbar"], t["wbar"], 0, G, P, K,
                                        t["q_scale"], t["k_scale"], t["qbar_scale"], want_bank=True)
    torch.cuda.synchronize()
    rows = _stratified(T, 64, always=np.arange(8176, 8212))
    h = _host(t)
    ri, rs, rb, _ = oracle.group_bank(h["q"], h["k"], h["w"], h["qbar"], h["wbar"], "fp8", 0, G, P, K,
                                      q_scale=h["q_scale"], k_scale=h["k_scale"], qbar_scale=h["qbar_scale"],
                                      rows=rows, want_bank=True)
    gbank = gb.cpu().numpy()
    exact = dist == "int"
    same = np.ones(len(rows), bool)
    for g in np.unique(rows // G):
        if exact:
            assert np.array_equal(gbank[g], rb[g]), g
            continue
        if (rb[g] == -1).all():
            assert (gbank[g] == -1).all()
            continue
        v = rb[g][rb[g] >= 0]
        brefs = pair_refs(h["qbar"], h["k"], h["wbar"], [g], "fp8", "fp8", h["qbar_scale"], h["k_scale"])
        _cmp(gbank[g:g + 1], None, rb[g:g + 1], brefs[0](0, v)[None, :], False, brefs, label=f"bank {g}")
        same[rows // G == g] = np.array_equal(gbank[g], rb[g])
    sel = np.nonzero(same)[0]
    _cmp(gi.cpu().numpy()[rows][sel], gs.cpu().numpy()[rows][sel], ri[sel], rs[sel], exact, _refs(h, "fp8", rows),
         sel=sel)
    other = rows[~same]
    if len(other):
        oi, osc = refine_over_bank(h, gbank, other, G, K, "fp8")
        _cmp(gi.cpu().numpy()[other], gs.cpu().numpy()[other], oi, osc, False, _refs(h, "fp8", other),
             label="own bank")


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
