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


# ------------------------------------------------------------------- rotary
# The rollout step's attention block (same page and section): before the
# scores, the new token's query and key head vectors are rotated by its
# position (rotary position embedding, the rotate-half form of the
# Qwen2.5-0.5B policy), the rotated key and the value are appended to the
# cache at that position, and attention runs over position + 1 cached
# positions.  For a head vector x of size D, pair i < D/2 is
# (x_i, x_{i+D/2}) and is turned by the angle pos * theta_i:
#     x'_i       = x_i cos - x_{i+D/2} sin
#     x'_{i+D/2} = x_{i+D/2} cos + x_i sin
# The library's definition computes this in binary32 with each product and
# the sum rounded separately, then rounds to bfloat16 (the cache format);
# rope_bf16 follows those steps, rope_f64 is the exact rotation.

def rope_f64(x, cos, sin):
    """x [..., D], cos / sin [..., D/2] broadcastable (binary64) -> rotated x."""
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16 bits (nearest, ties to even; finite
    inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def rope_bf16(x_bits, cos32, sin32):
    """x_bits [..., D] bfloat16 bits, cos32 / sin32 [..., D/2] binary32 ->
    bfloat16 bits of the rotation, each product and the sum rounded to
    binary32 (numpy's float32 arithmetic: IEEE single, no fused steps)."""
    x = (np.ascontiguousarray(x_bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    c, s = np.asarray(cos32, np.float32), np.asarray(sin32, np.float32)
    lo = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    hi = (b * c).astype(np.float32) + (a * s).astype(np.float32)
    return f32_to_bf16_bits(np.concatenate([lo, hi], axis=-1).astype(np.float32))


def decode_attention_rope(qkv_bits, cos32, sin32, pos, k_bits, v_bits, Hq, Hkv, scale):
    """The attention block of one decode step.  qkv_bits [S, (Hq + 2 Hkv) D]
    bfloat16 bits (query heads, then key heads, then value heads), cos32 /
    sin32 [Lmax, D/2] binary32 tables, pos [S], k_bits / v_bits
    [S, Hkv, Lmax, D] bfloat16 bits of the cache before the step.  Returns
    (out [S, Hq, D], lse [S, Hq], k_new, v_new): the binary64 attention of the
    rotated (bfloat16) queries over pos + 1 positions, and the caches after
    the append (bits).  A position outside [0, Lmax) appends nothing and its
    sequence's output is NaN (no cached key)."""
    S = qkv_bits.shape[0]
    Lmax, D = k_bits.shape[2], k_bits.shape[3]
    x = np.ascontiguousarray(qkv_bits, np.uint16).reshape(S, Hq + 2 * Hkv, D)
    k_new = np.array(k_bits, dtype=np.uint16, copy=True)
    v_new = np.array(v_bits, dtype=np.uint16, copy=True)
    q_rot = np.empty((S, Hq, D), np.uint16)
    lens = np.zeros(S, np.int64)
    for s in range(S):
        p = int(pos[s])
        ok = 0 <= p < Lmax
        cs = cos32[p] if ok else np.ones(D // 2, np.float32)
        sn = sin32[p] if ok else np.zeros(D // 2, np.float32)
        q_rot[s] = rope_bf16(x[s, :Hq], cs, sn)
        if ok:
            k_new[s, :, p] = rope_bf16(x[s, Hq:Hq + Hkv], cs, sn)
            v_new[s, :, p] = x[s, Hq + Hkv:]
            lens[s] = p + 1
    out, lse = decode_attention(bf16_to_f64(q_rot), bf16_to_f64(k_new), bf16_to_f64(v_new), lens,
                                scale)
    return out, lse, k_new, v_new
