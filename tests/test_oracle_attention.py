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
