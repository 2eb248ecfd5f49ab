"""The layer-wise dispatch on the GPU (Section 4.1 Eq. (5); Section 4.3;
Appendix C.4): one indexer_layers call runs layers with the four (G, P)
settings that Table 9 assigns to DeepSeek-V3.2's layers, (16, 8K), (8, 8K),
(16, 16K), (8, 16K), plus an original-indexer layer (G = 0), each on its own
inputs; every layer's banks and sampled rows match the oracle bit for bit
(integer inputs), and match a separate call of the same setting."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import compare
from workloads import make_workload

pytestmark = pytest.mark.gpu

TABLE9 = [(16, 8192), (8, 8192), (16, 16384), (8, 16384)]


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsa_amd as m
    m.lib()
    return m


def test_layers_table9_settings(dsa):
    T, K = 20480, 2048
    layers = []
    for n, (G, P) in enumerate(TABLE9 + [(0, 0)]):
        wl = make_workload(5, seed=100 + n, device="cuda", dist="int", T=T)
        t = wl.tensors
        L = dict(q=t["q"], k=t["k"], w=t["w"], G=G, P=P)
        if G == 16:
            L.update(qbar=t["qbar"], wbar=t["wbar"])
        elif G:  # the workload drew the group query for groups of 16: draw one per group of 8
            g = torch.Generator(device="cuda").manual_seed(200 + n)
            L["qbar"] = torch.randint(-3, 4, (T // G, 64, 128), generator=g, device="cuda").to(torch.bfloat16)
            L["wbar"] = torch.randint(-3, 4, (T // G, 64), generator=g, device="cuda").float()
        layers.append(L)
    outs = dsa.indexer_layers(layers, 0, K, want_score=True, want_bank=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.linspace(0, T - 1, 24).astype(np.int64), np.arange(T - 8, T),
                                     np.arange(8184, 8200), np.arange(16376, 16400)]))
    for (G, P), L, (gi, gs, gb) in zip(TABLE9 + [(0, 0)], layers, outs):
        h = {k: v.cpu() for k, v in L.items() if isinstance(v, torch.Tensor)}
        if G == 0:
            ri, rs = oracle.prefill(h["q"], h["k"], h["w"], "bf16", 0, K, rows=rows)
            compare(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, True, label="G=0")
            one, _ = dsa.indexer_prefill(L["q"], L["k"], L["w"], 0, K)
            assert torch.equal(one, gi)
            continue
        ri, rs, rb, pairs = oracle.group_bank(h["q"], h["k"], h["w"], h["qbar"], h["wbar"], "bf16", 0, G, P, K,
                                              rows=rows, want_bank=True)
        gbank = gb.cpu().numpy()
        for g in np.unique(rows // G):
            assert np.array_equal(gbank[g], rb[g]), (G, P, g)
        compare(gi.cpu().numpy()[rows], gs.cpu().numpy()[rows], ri, rs, True, label=f"G={G} P={P}")
        one, _, _ = dsa.indexer_group_bank(L["q"], L["k"], L["w"], L["qbar"], L["wbar"], 0, G, P, K)
        assert torch.equal(one, gi), (G, P)
