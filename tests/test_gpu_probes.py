"""The two measurement probes through the C ABI: the read stream returns the
XOR of every word it read, and the E4M3 matrix-core stream's accumulator sums
equal the sums of the products of its operands (so the rate it reports is a
rate of real 32x32x64 MFMAs)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_dsa_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("nbytes,nblocks", [(1 << 20, 7), ((1 << 20) + 13, 64), (100, 3)])
def test_read_probe_xor(dsa, nbytes, nblocks):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    out = dsa.read_probe(buf, nblocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    n16 = nbytes // 16
    words = host[:n16 * 16].view(np.uint32)
    want = np.bitwise_xor.reduce(words) if words.size else np.uint32(0)
    want ^= np.bitwise_xor.reduce(host[n16 * 16:].astype(np.uint32)) if nbytes % 16 else np.uint32(0)
    assert int(got) == int(want)


def _operands(mask, dtype):
    """The probe's operand words (a 32-bit mix of the word index under mask)
    as values [4 operands, 64 lanes, k]: a0, a1, b0, b1; each lane's operand
    is the first 8 (E4M3: 32 bytes) or 4 (bf16: 8 halves) words of its
    8-word slot."""
    h = np.arange(2048, dtype=np.uint32)
    with np.errstate(over="ignore"):
        h = h * np.uint32(0x9E3779B1)
        h ^= h >> np.uint32(15)
        h = h * np.uint32(0x85EBCA77)
        h ^= h >> np.uint32(13)
    words = (h & np.uint32(mask)).reshape(4, 64, 8)
    if dtype == "fp8":
        t = torch.from_numpy(words.copy().view(np.uint8)).view(torch.float8_e4m3fn)
        return t.float().numpy().reshape(4, 64, 32).astype(np.float64)
    halves = words[:, :, :4].copy().view(np.uint16)
    return torch.from_numpy(halves.view(np.int16)).view(torch.bfloat16).float().numpy().reshape(4, 64, 8).astype(
        np.float64)


@pytest.mark.parametrize("dtype,wps,mask", [("fp8", 1, 0x37373737), ("fp8", 2, 0x37373737),
                                            ("fp8", 4, 0x37373737), ("fp8", 2, 0x3E3E3E3E),
                                            ("bf16", 1, 0x3F7F3F7F), ("bf16", 4, 0x3F7F3F7F)])
def test_mfma_probe_sums(dsa, dtype, wps, mask):
    """A wave's 64 lane sums add up to the sum of all entries of its four
    accumulators, iters * sum over chains of sum_k colsum(A)[k] * rowsum(B)[k]:
    lane l holds row (A) or column (B) l % 32 and the k block l // 32."""
    ops = _operands(mask, dtype)
    kh = ops.shape[2]
    chains = [(0, 2), (1, 2), (0, 3), (1, 3)]  # (a, b) operand of accumulator c
    per_iter = 0.0
    for a, b in chains:
        for h in range(2):
            sa = ops[a, 32 * h:32 * h + 32].sum(axis=0)
            sb = ops[b, 32 * h:32 * h + 32].sum(axis=0)
            per_iter += float(sa[:kh] @ sb[:kh])
    nblocks = 5
    for iters in (1, 3):
        out, clocks = dsa.mfma_probe(iters, wps, nblocks, mask, dtype=dtype)
        torch.cuda.synchronize()
        lanes = out.cpu().numpy().astype(np.float64).reshape(nblocks * 4 * wps, 64)
        # the matrix core sums the products of each entry and the kernel 64
        # entries per lane in fp32: agreement to 1e-4 shows the products were
        # all taken
        np.testing.assert_allclose(lanes.sum(axis=1), iters * per_iter, rtol=1e-4)
        c = clocks.cpu().numpy()
        assert c.shape == (nblocks * 4 * wps, 2) and (c > 0).all()


def test_mfma_probe_rejects(dsa):
    with pytest.raises(Exception):
        dsa.mfma_probe(8, 3, 4)
    with pytest.raises(Exception):
        dsa.mfma_probe(8, 1, 4, 0xFFFFFFFF)
    with pytest.raises(Exception):
        dsa.mfma_probe(8, 1, 4, 0x7F807F80, dtype="bf16")
