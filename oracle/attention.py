"""CPU oracle of the decode-attention step (binary64).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline use it; the product path never imports it.

"Making Dr GRPO go brrr", section "What is RL post-training, and why is it
slow": the rollout phase runs one forward pass per generated token on a
(B*G, 1, hidden) input plus a growing KV cache, and the decode-attention
kernel the pages write replaces the scaled dot-product attention (SDPA) of
that step.  For sequence s and query head h, with the head's key/value
group g(h) = h // (Hq / Hkv) and the sequence's cached length len_s:

    x_j  = scale * <q[s, h], K[s, g, j]>            j < len_s
    o    = sum_j softmax(x)_j * V[s, g, j]

The definition is written out per (sequence, head) with numpy's binary64
matrix-vector products (library primitives) on the exactly widened bfloat16
inputs.  A sequence with no cached key (len_s < 1) has an empty softmax: its
output is NaN.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_attention(q, k, v, lens, scale):
    """q [S, Hq, D], k / v [S, Hkv, Lmax, D] (binary64), lens [S] ->
    (out [S, Hq, D], lse [S, Hq]) in binary64; lse = log sum_j exp(x_j)."""
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    out = np.empty((S, Hq, D))
    lse = np.empty((S, Hq))
    for s in range(S):
        L = int(lens[s])
        for h in range(Hq):
            g = h // grp
            if L < 1:
                out[s, h] = np.nan
                lse[s, h] = np.nan
                continue
            x = scale * (k[s, g, :L] @ q[s, h])
            m = x.max()
            p = np.exp(x - m)
            z = p.sum()
            out[s, h] = (p @ v[s, g, :L]) / z
            lse[s, h] = m + np.log(z)
    return out, lse
