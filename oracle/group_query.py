"""Oracle for the group indexer's query and gates (TEST INFRASTRUCTURE ONLY:
only tests, the smoke check and the benchmark's CPU leg use it).  numpy, fp64
arithmetic on the bf16 values the library feeds its matrix products.

"ADIndex: Layer-Adaptive Sparse Attention Indexing via Group-Level
Distillation" (Qi et al.), Section 4.2, Eq. (6)-(7), and Appendix C.3:

  cbar_t = W_pool [max_i c_i ; min_i c_i ; mean_i c_i]     (element-wise over
  hbar_t = mean_i h_i                                        the group's G rows)
  qbar_{t,j} = RoPE_t([W_Q cbar_t]_j),   wbar_{t,j} = sigmoid([W_G hbar_t]_j)

with the rotary embedding evaluated at the group anchor's position t.

Readings where the pages are silent: the pooled latents, cbar and hbar are
rounded to bf16 where they enter a bf16 product (the library's operand type);
the rotary embedding acts on the first `rope_dim` entries of each head, pairing
entry i with entry i + rope_dim/2 and turning it by t * base^(-2i/rope_dim);
the query is returned in bf16 (round to nearest even), the gates in fp32; only
complete groups get a query (the rows of an incomplete last group are zero).
"""
from __future__ import annotations

import numpy as np
import torch


def _bf16(x):
    """fp64/fp32 array -> nearest bf16 values (as float64)."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def _f64(t):
    return t.double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def pool(c, h, G):
    """Eq. (6) pooling of every complete group: ([max; min; mean] of c, mean of h)."""
    c, h = _f64(c), _f64(h)
    n = c.shape[0] // G
    cg = c[:n * G].reshape(n, G, -1)
    hg = h[:n * G].reshape(n, G, -1)
    return np.concatenate([cg.max(1), cg.min(1), cg.mean(1)], axis=1), hg.mean(1)


def rope(x, pos, rope_dim, base):
    """x [n, Hs, d] at positions pos [n]: rotate the pairs (i, i + rope_dim/2),
    i < rope_dim/2, of every head by pos * base^(-2i/rope_dim)."""
    x = np.array(x, np.float64)
    half = rope_dim // 2
    if half == 0:
        return x
    ang = np.asarray(pos, np.float64)[:, None] * base ** (-2.0 * np.arange(half) / rope_dim)  # [n, half]
    cos, sin = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half].copy(), x[..., half:rope_dim].copy()
    x[..., :half] = a * cos - b * sin
    x[..., half:rope_dim] = b * cos + a * sin
    return x


def group_query(c, h, w_pool, w_q, w_g, G, Hs, d, q_pos0=0, rope_dim=64, base=10000.0):
    """Eq. (6)-(7) for the complete groups of the rows of c [Tq, dc], h [Tq, dh]
    (queries at positions q_pos0 ..).  Returns (qbar float64 holding bf16 values
    [ceil(Tq/G), Hs, d], wbar float64 [ceil(Tq/G), Hs])."""
    Tq = c.shape[0]
    NG, n = -(-Tq // G), Tq // G
    pc, ph = pool(c, h, G)
    cbar = _bf16(_bf16(pc) @ _f64(w_pool).T)                # [n, dc]
    q = (cbar @ _f64(w_q).T).reshape(n, Hs, d)              # [n, Hs, d]
    anchors = q_pos0 + G * np.arange(n)
    q = _bf16(rope(q, anchors, rope_dim, base))
    g = _bf16(ph) @ _f64(w_g).T                             # [n, Hs]
    wb = 1.0 / (1.0 + np.exp(-g))
    qbar = np.zeros((NG, Hs, d))
    wbar = np.zeros((NG, Hs))
    qbar[:n], wbar[:n] = q, wb
    return qbar, wbar
