"""Pins of the decode-attention oracle against what does not depend on it:
torch's scaled_dot_product_attention (an independent library implementation
of the same definition, binary64 on the CPU), closed forms (one key, equal
keys), invariances of the definition (a common shift of the scores, a joint
permutation of keys and values) and the grouped-query head mapping."""
import numpy as np
import pytest

from oracle import attention as att
from synth.attention import get_decode_config, make_decode_case


def _f64(case):
    return att.bf16_to_f64(case.q), att.bf16_to_f64(case.k), att.bf16_to_f64(case.v)


@pytest.mark.parametrize("name", ["decode_ragged", "decode_mha_d128", "decode_gqa8"])
def test_against_torch_sdpa(name):
    import torch
    import torch.nn.functional as F

    cfg = get_decode_config(name)
    case = make_decode_case(cfg)
    q, k, v = _f64(case)
    out, lse = att.decode_attention(q, k, v, case.lens, cfg.scale)
    grp = cfg.Hq // cfg.Hkv
    for s in range(cfg.S):
        L = int(case.lens[s])
        Q = torch.tensor(q[s])[:, None, :]                      # [Hq, 1, D]
        K = torch.tensor(k[s, :, :L]).repeat_interleave(grp, 0)  # [Hq, L, D]
        V = torch.tensor(v[s, :, :L]).repeat_interleave(grp, 0)
        want = F.scaled_dot_product_attention(Q, K, V, scale=cfg.scale)[:, 0, :].numpy()
        assert np.abs(out[s] - want).max() <= 1e-13 * max(1.0, np.abs(want).max()), s


def test_one_key_returns_its_value():
    cfg = get_decode_config("decode_one_key")
    case = make_decode_case(cfg)
    q, k, v = _f64(case)
    out, lse = att.decode_attention(q, k, v, case.lens, cfg.scale)
    grp = cfg.Hq // cfg.Hkv
    for h in range(cfg.Hq):
        assert np.array_equal(out[:, h], v[:, h // grp, 0])
        assert np.allclose(lse[:, h], cfg.scale * np.einsum("sd,sd->s", q[:, h], k[:, h // grp, 0]),
                           rtol=0, atol=1e-14)


def test_equal_keys_give_the_mean_value():
    rng = np.random.default_rng(3)
    S, Hq, Hkv, L, D = 2, 4, 2, 37, 16
    q = rng.normal(size=(S, Hq, D))
    k = np.repeat(rng.normal(size=(S, Hkv, 1, D)), L, axis=2)
    v = rng.normal(size=(S, Hkv, L, D))
    out, lse = att.decode_attention(q, k, v, np.full(S, L), 0.25)
    want = np.repeat(v.mean(axis=2), Hq // Hkv, axis=1)
    assert np.abs(out - want).max() < 1e-14


def test_score_shift_and_permutation_invariance():
    cfg = get_decode_config("decode_ragged")
    case = make_decode_case(cfg)
    q, k, v = _f64(case)
    out, lse = att.decode_attention(q, k, v, case.lens, cfg.scale)
    # a common shift of every key by c moves all scores of a head by the same
    # amount (scale * <q, c>): the output does not change
    c = np.random.default_rng(4).normal(size=(cfg.S, cfg.Hkv, 1, cfg.D))
    out2, _ = att.decode_attention(q, k + c, v, case.lens, cfg.scale)
    assert np.abs(out2 - out).max() < 1e-11
    # permuting the cached positions of keys and values together
    k3, v3 = k.copy(), v.copy()
    for s in range(cfg.S):
        L = int(case.lens[s])
        p = np.random.default_rng(s).permutation(L)
        k3[s, :, :L] = k[s][:, p]
        v3[s, :, :L] = v[s][:, p]
    out3, lse3 = att.decode_attention(q, k3, v3, case.lens, cfg.scale)
    assert np.abs(out3 - out).max() < 1e-12 and np.abs(lse3 - lse).max() < 1e-12


def test_softmax_normalises():
    """exp(x_j - lse) over the cached keys sums to 1."""
    cfg = get_decode_config("decode_gqa8")
    case = make_decode_case(cfg)
    q, k, v = _f64(case)
    _, lse = att.decode_attention(q, k, v, case.lens, cfg.scale)
    grp = cfg.Hq // cfg.Hkv
    for s in range(cfg.S):
        L = int(case.lens[s])
        for h in range(cfg.Hq):
            x = cfg.scale * (k[s, h // grp, :L] @ q[s, h])
            assert abs(np.exp(x - lse[s, h]).sum() - 1.0) < 1e-12


def test_grouped_query_head_mapping():
    """Query head h reads key/value head h // (Hq / Hkv): changing key/value
    head 1 changes exactly the query heads of group 1."""
    cfg = get_decode_config("decode_gqa8")
    case = make_decode_case(cfg)
    q, k, v = _f64(case)
    out, _ = att.decode_attention(q, k, v, case.lens, cfg.scale)
    v2 = v.copy()
    v2[:, 1] += 1.0
    out2, _ = att.decode_attention(q, k, v2, case.lens, cfg.scale)
    grp = cfg.Hq // cfg.Hkv
    changed = np.abs(out2 - out).max(axis=(0, 2)) > 0
    assert changed.tolist() == [h // grp == 1 for h in range(cfg.Hq)]
    # softmax weights sum to one, so adding 1 to every value adds exactly 1
    assert np.abs(out2[:, grp:2 * grp] - out[:, grp:2 * grp] - 1.0).max() < 1e-12


def test_empty_cache_is_nan():
    q = np.ones((1, 2, 4))
    k = np.ones((1, 1, 3, 4))
    out, lse = att.decode_attention(q, k, k, np.array([0]), 0.5)
    assert np.isnan(out).all() and np.isnan(lse).all()


# ---------------------------------------------------------------- rotary
def _tables(Lmax, D, base=1.0e6):
    inv = 1.0 / base ** (np.arange(0, D // 2, dtype=np.float64) / (D // 2))
    ang = np.arange(Lmax, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 5, 64))
    c, s = _tables(4, 64)
    assert np.array_equal(att.rope_f64(x, c[0], s[0]), x)
    bits = att.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(att.rope_bf16(bits, c[0].astype(np.float32), s[0].astype(np.float32)),
                          bits)


def test_rope_is_a_complex_rotation_of_each_pair():
    """Pair i of the rotate-half form, (x_i, x_{i+D/2}), read as the complex
    number x_i + 1j x_{i+D/2}, is multiplied by exp(1j * angle_i)."""
    rng = np.random.default_rng(12)
    D = 64
    x = rng.standard_normal((7, D))
    c, s = _tables(100, D)
    p = 37
    z = (x[:, :D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * np.arctan2(s[p], c[p]))
    want = np.concatenate([z.real, z.imag], axis=-1)
    assert np.abs(att.rope_f64(x, c[p], s[p]) - want).max() <= 1e-14


def test_rope_relative_position():
    """Scores of rotated queries and keys depend on the positions only through
    their difference (and rotation keeps each pair's length)."""
    rng = np.random.default_rng(13)
    D = 128
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    c, s = _tables(4096, D)
    a = att.rope_f64(q, c[5], s[5]) @ att.rope_f64(k, c[2], s[2])
    b = att.rope_f64(q, c[3005], s[3005]) @ att.rope_f64(k, c[3002], s[3002])
    assert abs(a - b) <= 1e-11 * (np.abs(q) @ np.abs(k))
    r = att.rope_f64(q, c[700], s[700])
    n = q[:D // 2] ** 2 + q[D // 2:] ** 2
    assert np.abs(r[:D // 2] ** 2 + r[D // 2:] ** 2 - n).max() <= 1e-13 * n.max()


def test_rope_bf16_is_the_rotation_rounded():
    """The binary32-then-bfloat16 steps stay within one bfloat16 rounding (plus
    the binary32 ones) of the exact rotation of the same inputs."""
    rng = np.random.default_rng(14)
    D = 64
    x32 = rng.standard_normal((50, D)).astype(np.float32)
    bits = att.f32_to_bf16_bits(x32)
    xs = att.bf16_to_f64(bits)
    c, s = _tables(2048, D)
    for p in (1, 17, 1999):
        c32, s32 = c[p].astype(np.float32), s[p].astype(np.float32)
        got = att.bf16_to_f64(att.rope_bf16(bits, c32, s32))
        want = att.rope_f64(xs, c32.astype(np.float64), s32.astype(np.float64))
        scale = np.abs(xs).max()
        assert (np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6 * scale).all(), p


def test_f32_to_bf16_rounding():
    """Nearest-even rounding to bfloat16 against the exact halfway cases."""
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5,
                     1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    got = att.bf16_to_f64(att.f32_to_bf16_bits(vals))
    # ties go to the even neighbour; 1 + 2^-9 is below half an ulp
    want = np.array([1.0, 1.0, 1.0 + 4 * 2.0 ** -8, 1.0, -2.5, 1.0 + 2 * 2.0 ** -8])
    assert np.array_equal(got, want)


def test_decode_attention_rope_block():
    """The block appends the rotated key and the value at each sequence's
    position (nothing else in the cache changes), attends over position + 1
    positions with the rotated query, and leaves a sequence whose position is
    outside the cache untouched with a NaN output."""
    rng = np.random.default_rng(15)
    S, Hq, Hkv, D, Lmax = 5, 4, 2, 64, 24
    pos = np.array([0, 3, 23, 11, 24])
    qkv = att.f32_to_bf16_bits(rng.standard_normal((S, (Hq + 2 * Hkv) * D)).astype(np.float32))
    k0 = att.f32_to_bf16_bits(rng.standard_normal((S, Hkv, Lmax, D)).astype(np.float32))
    v0 = att.f32_to_bf16_bits(rng.standard_normal((S, Hkv, Lmax, D)).astype(np.float32))
    c, s = _tables(Lmax, D)
    c32, s32 = c.astype(np.float32), s.astype(np.float32)
    out, lse, k1, v1 = att.decode_attention_rope(qkv, c32, s32, pos, k0, v0, Hq, Hkv, 0.125)
    x = qkv.reshape(S, Hq + 2 * Hkv, D)
    for i in range(S):
        p = int(pos[i])
        changed = np.zeros(Lmax, bool)
        if p < Lmax:
            changed[p] = True
            assert np.array_equal(v1[i, :, p], x[i, Hq + Hkv:])
            assert np.array_equal(k1[i, :, p], att.rope_bf16(x[i, Hq:Hq + Hkv], c32[p], s32[p]))
            q = att.bf16_to_f64(att.rope_bf16(x[i, :Hq], c32[p], s32[p]))
            want, _ = att.decode_attention(q[None], att.bf16_to_f64(k1[i:i + 1]),
                                           att.bf16_to_f64(v1[i:i + 1]), [p + 1], 0.125)
            assert np.array_equal(out[i], want[0])
        else:
            assert np.isnan(out[i]).all()
        assert np.array_equal(k1[i][:, ~changed], k0[i][:, ~changed])
        assert np.array_equal(v1[i][:, ~changed], v0[i][:, ~changed])
