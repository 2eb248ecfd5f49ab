"""Seeded generators for the indexer workloads.

The prefill tensors are drawn from one ``torch.Generator`` seeded with the
workload's seed, in a fixed order (q, k, w; for decode q, cache, w).  The
group-indexer q-bar and w-bar come from a second generator seeded with
seed + 0x9E3779B1, so a group-bank workload's q, k and w are the same bytes as
the prefill workload of the same seed.  The same seed on the same device always gives the same
bytes; the CPU and GPU random streams differ, so the oracle always consumes a
host copy of exactly the bytes the GPU path consumed.

Byte formats (all row-major, last dimension fastest):

* bf16 tensors are ``torch.bfloat16`` (round-to-nearest-even from fp32);
* fp8 tensors are ``torch.uint8`` codes of OCP FP8 E4M3 (the "fn" variant:
  bias 7, no infinities, max 448) with one fp32 scale per token.  A token's
  scale is amax/448 over its values (all heads for a query token, the d values
  for a key token); an all-zero token gets scale 1.  Codes are
  round-to-nearest-even of value/scale, clamped to +-448 first;
* fp32 tensors are ``torch.float32``.

Integer-valued variants keep every value an integer in a small range so that
every fp32 partial sum of the indexer score is exact: for fp8 these use scale 1
(every integer in [-3, 3] is an exact E4M3 code).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

E4M3_MAX = 448.0

# The five workload shapes.  "int" marks integer-valued inputs.
CONFIGS = {
    # tiny prefill: T=1024, H=4, d=32, top-k 64, integer inputs, w in [0, 3]
    1: dict(kind="prefill", T=1024, H=4, d=32, topk=64, dtype="bf16", dist="int", w_lo=0, w_hi=3),
    # DSA-shaped prefill, one layer, bf16
    2: dict(kind="prefill", T=16384, H=64, d=128, topk=2048, dtype="bf16", dist="normal"),
    # long prefill, one layer, fp8 with per-token scales, query chunks of 4096
    3: dict(kind="prefill", T=131072, H=64, d=128, topk=2048, dtype="fp8", dist="normal", chunk=4096),
    # decode scan: 32 sequences x 262144 cached keys, fp8 cache, bf16 query
    4: dict(kind="decode", B=32, N=262144, H=64, d=128, topk=2048, dist="normal"),
    # ADIndex group token bank: T=65536, G=16, P=8192, group indexer with 64 heads
    5: dict(kind="group_bank", T=65536, H=64, Hs=64, d=128, topk=2048, G=16, P=8192,
            dtype="bf16", dist="normal"),
}


@dataclass
class Workload:
    kind: str
    dtype: str
    params: dict
    tensors: dict = field(default_factory=dict)

    def __getitem__(self, name):
        return self.tensors[name]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(g, shape, device, std=1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _ints(g, shape, lo, hi, device) -> torch.Tensor:
    return torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int32).to(torch.float32)


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16, round to nearest even."""
    return x.to(torch.bfloat16)


def e4m3_quantize_rows(x: torch.Tensor, unit_scale: bool = False):
    """Quantise fp32 ``x[..., n]`` to E4M3 codes with one fp32 scale per row.

    Returns ``(codes uint8 [..., n], scale float32 [...])``.  With
    ``unit_scale`` the scale is 1 (for integer-valued inputs that are exact
    E4M3 values already).
    """
    if unit_scale:
        scale = torch.ones(x.shape[:-1], dtype=torch.float32, device=x.device)
        y = x
    else:
        amax = x.abs().amax(dim=-1)
        scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        y = x / scale.unsqueeze(-1)
    y = y.clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def _qk(g, shape, dist, dtype, device, std):
    """Draw one q or k tensor in the requested format; returns (data, scale|None)."""
    if dist == "int":
        x = _ints(g, shape, -3, 3, device)
    else:
        x = _normal(g, shape, device, std if dtype == "bf16" else 1.0)
    if dtype == "bf16":
        return to_bf16(x).contiguous(), None
    if dtype == "fp8":
        # a query token's scale spans all of its heads: quantise [T, H*d] rows
        flat = x.reshape(shape[0], -1)
        codes, scale = e4m3_quantize_rows(flat, unit_scale=(dist == "int"))
        return codes.reshape(shape), scale
    raise ValueError(dtype)


def _weights(g, shape, dist, device, H, w_lo=-3, w_hi=3):
    if dist == "int":
        return _ints(g, shape, w_lo, w_hi, device)
    return _normal(g, shape, device, 1.0 / math.sqrt(H))


def make_prefill(T, H, d, topk, dtype="bf16", dist="normal", seed=0, device="cpu",
                 Tq=None, q_pos0=None, w_lo=-3, w_hi=3, **_):
    """Prefill inputs: q [Tq,H,d], k [T,d], w [Tq,H]; queries at q_pos0..q_pos0+Tq-1.

    With ``Tq`` smaller than ``T`` the queries are the last ``Tq`` positions
    unless ``q_pos0`` says otherwise.
    """
    Tq = T if Tq is None else Tq
    q_pos0 = T - Tq if q_pos0 is None else q_pos0
    g = _gen(seed, device)
    std = 1.0 / math.sqrt(d)
    q, q_scale = _qk(g, (Tq, H, d), dist, dtype, device, std)
    k, k_scale = _qk(g, (T, d), dist, dtype, device, std)
    w = _weights(g, (Tq, H), dist, device, H, w_lo, w_hi).contiguous()
    t = dict(q=q, k=k, w=w)
    if dtype == "fp8":
        t.update(q_scale=q_scale, k_scale=k_scale)
    return Workload("prefill", dtype, dict(T=T, Tq=Tq, Tk=T, H=H, d=d, topk=topk, q_pos0=q_pos0,
                                           dist=dist, seed=seed), t)


def make_decode(B, N, H, d, topk, dist="normal", seed=0, device="cpu", seq_lens=None,
                w_lo=-3, w_hi=3, **_):
    """Decode inputs: q [B,H,d] bf16, fp8 cache [B,N,d] + scale [B,N], w [B,H], seq_lens [B]."""
    g = _gen(seed, device)
    if dist == "int":
        q = to_bf16(_ints(g, (B, H, d), -3, 3, device)).contiguous()
        kc = _ints(g, (B * N, d), -3, 3, device)
        codes, scale = e4m3_quantize_rows(kc, unit_scale=True)
    else:
        q = to_bf16(_normal(g, (B, H, d), device)).contiguous()
        codes = torch.empty((B * N, d), dtype=torch.uint8, device=device)
        scale = torch.empty((B * N,), dtype=torch.float32, device=device)
        step = 1 << 20
        for r0 in range(0, B * N, step):  # bounded fp32 temporaries
            r1 = min(B * N, r0 + step)
            c, s = e4m3_quantize_rows(_normal(g, (r1 - r0, d), device))
            codes[r0:r1] = c
            scale[r0:r1] = s
    w = _weights(g, (B, H), dist, device, H, w_lo, w_hi).contiguous()
    if seq_lens is None:
        seq_lens = torch.full((B,), N, dtype=torch.int32, device=device)
    else:
        seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32, device=device)
    t = dict(q=q, k_cache=codes.reshape(B, N, d), k_scale=scale.reshape(B, N), w=w, seq_lens=seq_lens)
    return Workload("decode", "fp8", dict(B=B, N=N, H=H, d=d, topk=topk, dist=dist, seed=seed), t)


def make_group_bank(T, H, Hs, d, topk, G, P, dtype="bf16", dist="normal", seed=0, device="cpu",
                    Tq=None, q_pos0=None, w_lo=-3, w_hi=3, **_):
    """Group-bank inputs: the prefill inputs plus q-bar [NG,Hs,d] and w-bar [NG,Hs].

    q-bar and w-bar stand in for the group query and gate projections of a
    trained group indexer: q-bar is drawn like q; w-bar is a sigmoid of a
    standard normal, as the group gate is a sigmoid (integer variant: w-bar
    integers).
    """
    wl = make_prefill(T, H, d, topk, dtype, dist, seed, device, Tq, q_pos0, w_lo, w_hi)
    Tq = wl.params["Tq"]
    NG = -(-Tq // G)
    g = _gen(seed + 0x9E3779B1, device)
    qbar, qbar_scale = _qk(g, (NG, Hs, d), dist, dtype, device, 1.0 / math.sqrt(d))
    if dist == "int":
        wbar = _ints(g, (NG, Hs), w_lo, w_hi, device)
    else:
        wbar = torch.sigmoid(_normal(g, (NG, Hs), device))
    wl.tensors.update(qbar=qbar, wbar=wbar.contiguous())
    if dtype == "fp8":
        wl.tensors["qbar_scale"] = qbar_scale
    wl.kind = "group_bank"
    wl.params.update(Hs=Hs, G=G, P=P, NG=NG)
    return wl


def make_mtp(B, N, m, H, Hs, d, topk, G, P, dist="normal", seed=0, device="cpu", prefix_lens=None,
             w_lo=-3, w_hi=3, **_):
    """MTP verification inputs: the decode cache (E4M3 [B,N,d] + scale [B,N]),
    m bf16 queries per sequence q [B,m,H,d], w [B,m,H], the group indexer's
    q-bar [B,m/G,Hs,d] bf16 and w-bar [B,m/G,Hs] (drawn as in the group bank
    inputs), and prefix_lens [B] int32: the keys the window's first query sees
    (default N - m + 1, so the last query sees the whole cache)."""
    wl = make_decode(B * m, 1, H, d, topk, dist, seed, device, w_lo=w_lo, w_hi=w_hi)  # queries and gates
    kv = make_decode(B, N, 1, d, topk, dist, seed + 1, device)                        # the caches
    g = _gen(seed + 0x9E3779B1, device)
    NGs = m // G
    if dist == "int":
        qbar = to_bf16(_ints(g, (B, NGs, Hs, d), -3, 3, device)).contiguous()
        wbar = _ints(g, (B, NGs, Hs), w_lo, w_hi, device)
    else:
        qbar = to_bf16(_normal(g, (B, NGs, Hs, d), device)).contiguous()
        wbar = torch.sigmoid(_normal(g, (B, NGs, Hs), device))
    if prefix_lens is None:
        prefix_lens = torch.full((B,), N - m + 1, dtype=torch.int32, device=device)
    else:
        prefix_lens = torch.as_tensor(prefix_lens, dtype=torch.int32, device=device)
    t = dict(q=wl["q"].reshape(B, m, H, d).contiguous(), w=wl["w"].reshape(B, m, H).contiguous(),
             k_cache=kv["k_cache"], k_scale=kv["k_scale"], qbar=qbar, wbar=wbar.contiguous(),
             prefix_lens=prefix_lens)
    return Workload("mtp", "fp8", dict(B=B, N=N, m=m, H=H, Hs=Hs, d=d, topk=topk, G=G, P=P, dist=dist,
                                       seed=seed), t)


def make_workload(config: int, seed: int = 0, device="cpu", dist=None, **override):
    """The workload of one of the five configurations (optionally resized)."""
    p = dict(CONFIGS[config])
    if dist is not None:
        p["dist"] = dist
    p.update(override)
    kind = p.pop("kind")
    if kind == "prefill":
        return make_prefill(seed=seed, device=device, **p)
    if kind == "decode":
        return make_decode(seed=seed, device=device, **p)
    return make_group_bank(seed=seed, device=device, **p)
