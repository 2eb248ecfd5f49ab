"""The decode entry point that allocates nothing (indexer_decode_noalloc): its
workspace is the library's fixed device scratch array.  Through the C ABI,
two calls in a row (the second smaller, so it runs over what the first left
in the scratch) must match indexer_decode with a caller workspace bit for
bit (same kernels); sizes beyond the scratch are refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

from workloads import make_decode

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_dsa_amd import _lib
    return _lib.lib()


def _noalloc(L, t, K):
    B, H, d = t["q"].shape
    N = t["k_cache"].shape[1]
    idx = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, K), 7.0, dtype=torch.float32, device="cuda")
    rc = L.indexer_decode_noalloc(t["q"].data_ptr(), t["k_cache"].data_ptr(), t["k_scale"].data_ptr(),
                                  t["w"].data_ptr(), t["seq_lens"].data_ptr(), B, N, H, d, K, idx.data_ptr(),
                                  sc.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, L.indexer_last_error().decode()
    return idx, sc


def test_noalloc_matches_decode_twice(L):
    import sparse_attention_indexer_dsa_amd as dsa
    cases = [dict(B=6, N=20000, K=512, seq=[20000, 1, 777, 19999, 4096, 300], seed=1),
             dict(B=2, N=3000, K=128, seq=[3000, 50], seed=2)]
    for c in cases:
        wl = make_decode(c["B"], c["N"], 64, 128, c["K"], dist="normal", seed=c["seed"], seq_lens=c["seq"])
        t = {k: v.cuda() for k, v in wl.tensors.items()}
        ref_i, ref_s = dsa.indexer_decode(t["q"], t["k_cache"], t["k_scale"], t["w"], t["seq_lens"], c["K"])
        got_i, got_s = _noalloc(L, t, c["K"])
        torch.cuda.synchronize()
        assert torch.equal(ref_i, got_i), c
        assert torch.equal(ref_s, got_s), c
        for b, n in enumerate(c["seq"]):  # valid entries then padding
            assert (got_i[b] >= 0).sum().item() == min(n, c["K"])


def test_noalloc_refuses_beyond_scratch(L):
    cap = L.indexer_decode_noalloc_max_bytes()
    assert cap == 96 << 20
    p = ctypes.c_void_p(1 << 20)
    rc = L.indexer_decode_noalloc(p, p, p, p, p, 64, 262144, 64, 128, 2048, p, None, None)
    assert rc == -2 and "scratch" in L.indexer_last_error().decode()
