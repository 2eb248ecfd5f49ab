"""Randomized parity sweep: seeded random shapes across the supported range of
every entry point (dtype, heads, head dim, top-k, query offsets, ragged
decode lengths, group size and bank budget), each checked against the oracle
on sampled rows.  Integer inputs are compared exactly, normal inputs under
the tolerance rule.  The shapes stay small enough for the oracle to finish in
seconds, yet they span several tiles, ragged tails and rows shorter than K."""
import numpy as np
import pytest
import torch

from tests.test_gpu_parity import _decode_check, _group_check, _prefill_check, _rows
from workloads import make_decode, make_group_bank, make_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsa_amd as m
    m.lib()
    return m


def _prefill_case(i):
    r = np.random.default_rng(1000 + i)
    dtype = ["bf16", "fp8"][i % 2]
    d = int(r.choice([64, 128] if dtype == "fp8" else [32, 64, 128]))
    H = int(r.choice([1, 3, 8, 17, 32, 33, 48, 63, 64]))
    T = int(r.integers(1, 2500))
    Tq = int(r.integers(1, T + 1))
    q_pos0 = int(r.integers(0, T - Tq + 1))
    topk = int(r.choice([1, 7, 64, 300, 1024, 2048]))
    dist = ["int", "normal"][(i // 2) % 2]
    return dict(T=T, H=H, d=d, topk=topk, dtype=dtype, dist=dist, seed=i, Tq=Tq, q_pos0=q_pos0)


def _decode_case(i):
    r = np.random.default_rng(2000 + i)
    B = int(r.integers(1, 40))
    N = int(r.integers(1, 6000))
    H = int(r.choice([1, 5, 16, 32, 40, 64]))
    d = int(r.choice([64, 128]))
    topk = int(r.choice([1, 33, 256, 2048]))
    lens = [int(x) for x in r.integers(0, N + 1, B)]
    dist = ["int", "normal"][i % 2]
    return dict(B=B, N=N, H=H, d=d, topk=topk, dist=dist, seed=i, seq_lens=lens)


def _group_case(i):
    """(inputs, flags): every third case pools the group's own queries
    (bf16, Hs = H), every third forces the bank for every complete group."""
    r = np.random.default_rng(3000 + i)
    G = int(r.choice([4, 8, 16]))
    topk = int(r.choice([16, 64, 256]))
    P = int(r.choice([topk, topk + 5, 2 * topk, 1000]))
    T = int(r.integers(P // 2, 3000))
    Tq = int(r.integers(1, T + 1))
    q_pos0 = (int(r.integers(0, T - Tq + 1)) // G) * G
    H = int(r.choice([8, 33, 64]))
    Hs = int(r.choice([1, 8, H]))
    dtype = ["bf16", "fp8"][i % 2]
    flags = 0
    if i % 3 == 0:
        dtype, Hs, flags = "bf16", H, "pool"
    elif i % 3 == 1:
        flags = "force"
    dist = "normal" if i % 4 == 3 else "int"
    return dict(T=T, H=H, Hs=Hs, d=128, topk=topk, G=G, P=P, dtype=dtype, dist=dist, seed=i, Tq=Tq,
                q_pos0=q_pos0), flags


@pytest.mark.parametrize("i", range(48))
def test_sweep_prefill(dsa, i):
    c = _prefill_case(i)
    wl = make_prefill(**c)
    _prefill_check(dsa, wl, rows=_rows(c["Tq"], 64, seed=i))


@pytest.mark.parametrize("i", range(24))
def test_sweep_decode(dsa, i):
    c = _decode_case(i)
    wl = make_decode(**c)
    _decode_check(dsa, wl)


@pytest.mark.parametrize("i", range(24))
def test_sweep_group_bank(dsa, i):
    c, how = _group_case(i)
    wl = make_group_bank(**c)
    flags = {0: 0, "pool": dsa.POOL_MEAN, "force": dsa.FORCE_BANK}[how]
    _group_check(dsa, wl, flags=flags, rows=_rows(c["Tq"], 48, seed=i))
