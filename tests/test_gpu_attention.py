"""GPU parity of the decode-attention step against the binary64 oracle:
every output element and log-sum-exp on ragged caches, one-key caches, two
head geometries and the full rollout decode shape (B*G = 64 sequences,
14 query / 2 key-value heads of size 64, 512 and 1024 cached positions).

Tolerance: the output is bfloat16 rounded from a binary32 computation, so
|got - want| <= 2^-8 |want| + 2^-12 max|V| (one rounding of a value whose
binary32 accumulation over at most a few thousand weighted values is good
to well below 2^-12 of the values' scale); the log-sum-exp (binary32)
within 2e-5 absolute."""
import numpy as np
import pytest
import torch

import rl_post_loss_dr_amd as dr
from oracle import attention as att
from synth.attention import get_decode_config, make_decode_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _run(case, lens=None, scale=None):
    c = case.cfg
    lens = case.lens if lens is None else lens
    out, lse = dr.decode_attention(_dev_bf16(case.q), _dev_bf16(case.k), _dev_bf16(case.v),
                                   torch.from_numpy(np.ascontiguousarray(lens, np.int32)).to(DEV),
                                   scale=c.scale if scale is None else scale, want_lse=True)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(case, got, lse, lens=None, scale=None):
    c = case.cfg
    lens = case.lens if lens is None else lens
    q, k, v = (att.bf16_to_f64(x) for x in (case.q, case.k, case.v))
    want, want_lse = att.decode_attention(q, k, v, lens, c.scale if scale is None else scale)
    bound = 2.0 ** -8 * np.abs(want) + 2.0 ** -12 * np.abs(v).max()
    err = np.abs(got - want)
    assert (err <= bound).all(), float((err - bound).max())
    assert np.abs(lse - want_lse).max() <= 2e-5, float(np.abs(lse - want_lse).max())
    return float(err.max())


@pytest.mark.parametrize("name", ["decode_ragged", "decode_one_key", "decode_mha_d128",
                                  "decode_gqa8", "decode_gqa16_d128", "decode_s64_l512",
                                  "decode_s64_l1024", "decode_s256_l1024", "decode_long_d64",
                                  "decode_long_d128"])
def test_decode_attention_parity(name):
    print(f"case {name}", flush=True)
    case = make_decode_case(get_decode_config(name))
    got, lse = _run(case)
    _check(case, got, lse)


def test_decode_attention_deterministic_and_scale():
    case = make_decode_case(get_decode_config("decode_gqa8"))
    a1, l1 = _run(case)
    a2, l2 = _run(case)
    assert np.array_equal(a1, a2) and np.array_equal(l1, l2)
    got, lse = _run(case, scale=0.3)
    _check(case, got, lse, scale=0.3)


def test_decode_attention_length_edges():
    """len 0 gives NaN (empty softmax); lengths above the capacity count as
    the capacity; len 1 returns the first cached value."""
    case = make_decode_case(get_decode_config("decode_ragged"))
    c = case.cfg
    lens = case.lens.copy()
    lens[1] = 0
    lens[2] = c.Lmax + 50
    got, lse = _run(case, lens=lens)
    assert np.isnan(got[1]).all() and np.isnan(lse[1]).all()
    ref_lens = lens.copy()
    ref_lens[2] = c.Lmax
    keep = np.ones(c.S, bool)
    keep[1] = False
    q, k, v = (att.bf16_to_f64(x) for x in (case.q, case.k, case.v))
    want, _ = att.decode_attention(q[keep], k[keep], v[keep], ref_lens[keep], c.scale)
    bound = 2.0 ** -8 * np.abs(want) + 2.0 ** -12 * np.abs(v).max()
    assert (np.abs(got[keep] - want) <= bound).all()
    one = lens.copy()
    one[:] = 1
    got1, _ = _run(case, lens=one)
    grp = c.Hq // c.Hkv
    for h in range(c.Hq):
        assert np.array_equal(got1[:, h], att.bf16_to_f64(case.v)[:, h // grp, 0])


def test_decode_attention_reused_workspace():
    """One workspace serves many calls (results identical call after call,
    also across different cache lengths)."""
    case = make_decode_case(get_decode_config("decode_gqa8"))
    c = case.cfg
    q, k, v = _dev_bf16(case.q), _dev_bf16(case.k), _dev_bf16(case.v)
    ws = torch.empty(dr.decode_attention_workspace_bytes(c.S, c.Hq, c.Hkv, c.Lmax, c.D),
                     dtype=torch.uint8, device=DEV)
    lens = torch.from_numpy(case.lens).to(DEV)
    first = dr.decode_attention(q, k, v, lens, workspace=ws).clone()
    short = torch.clamp(lens, max=70)
    for _ in range(3):
        dr.decode_attention(q, k, v, short, workspace=ws)
        again = dr.decode_attention(q, k, v, lens, workspace=ws)
        assert torch.equal(again, first)
    torch.cuda.synchronize()
    got = first.float().cpu().numpy().astype(np.float64)
    _, want_lse = att.decode_attention(*(att.bf16_to_f64(x) for x in (case.q, case.k, case.v)),
                                       case.lens, c.scale)
    assert got.shape == (c.S, c.Hq, c.D) and np.isfinite(want_lse).all()


@pytest.mark.parametrize("name", ["decode_s64_l512", "decode_gqa8"])
def test_decode_attention_graph_replay(name):
    """The decode step replayed from a captured graph (as a decode loop, and
    the benchmark, issue it): every replay equals the eager result, with eager
    work and synchronisations between replays.  decode_gqa8 takes the split
    path (fused kernel + combine), decode_s64_l512 the single kernel."""
    print(f"case {name}", flush=True)
    case = make_decode_case(get_decode_config(name))
    c = case.cfg
    q, k, v = _dev_bf16(case.q), _dev_bf16(case.k), _dev_bf16(case.v)
    lens = torch.from_numpy(np.ascontiguousarray(case.lens, np.int32)).to(DEV)
    ws = torch.empty(dr.decode_attention_workspace_bytes(c.S, c.Hq, c.Hkv, c.Lmax, c.D),
                     dtype=torch.uint8, device=DEV)
    eager = dr.decode_attention(q, k, v, lens, workspace=ws).clone()
    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dr.decode_attention(q, k, v, lens, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dr.decode_attention(q, k, v, lens, workspace=ws, out=out)
    short = torch.clamp(lens, max=40)
    for _ in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        other = dr.decode_attention(q, k, v, short, workspace=ws)  # eager work in between
        torch.cuda.synchronize()
        assert other.shape == eager.shape


def _rope_tables(Lmax, D, base=1.0e6):
    inv = 1.0 / base ** (np.arange(0, D // 2, dtype=np.float64) / (D // 2))
    ang = np.arange(Lmax, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _bf16_bits(rng_seed, shape, std=1.0):
    g = torch.Generator().manual_seed(rng_seed)
    t = (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("S,Hq,Hkv,D,Lmax", [(64, 14, 2, 64, 512), (8, 16, 2, 128, 300),
                                            (5, 4, 4, 64, 40)])
def test_decode_attention_rope_parity(S, Hq, Hkv, D, Lmax):
    """Rotary embedding + cache append + attention against the oracle: the
    appended cache entries bit for bit (every other entry unchanged), the
    output and log-sum-exp within the attention tolerance; positions 0,
    Lmax - 1 and (small case) outside the cache."""
    print(f"case S={S} Hq={Hq} Hkv={Hkv} D={D} Lmax={Lmax}", flush=True)
    rng = np.random.default_rng(S * 1000 + D + Lmax)
    pos = rng.integers(0, Lmax, S).astype(np.int32)
    pos[0], pos[-1] = 0, Lmax - 1
    if S >= 5 and Lmax == 40:
        pos[1], pos[2] = Lmax, -1  # outside the cache: no append, NaN output
    qkv = _bf16_bits(S + D, (S, (Hq + 2 * Hkv) * D))
    k0 = _bf16_bits(S + D + 1, (S, Hkv, Lmax, D))
    v0 = _bf16_bits(S + D + 2, (S, Hkv, Lmax, D))
    cos, sin = _rope_tables(Lmax, D)
    scale = 1.0 / np.sqrt(D)
    kc, vc = _dev_bf16(k0), _dev_bf16(v0)
    out, lse = dr.decode_attention_rope(
        _dev_bf16(qkv), torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV),
        torch.from_numpy(pos).to(DEV), kc, vc, Hq, scale=scale, want_lse=True)
    torch.cuda.synchronize()
    want, want_lse, k1, v1 = att.decode_attention_rope(qkv, cos, sin, pos, k0, v0, Hq, Hkv, scale)
    assert np.array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), k1)
    assert np.array_equal(vc.view(torch.int16).cpu().numpy().view(np.uint16), v1)
    got = out.float().cpu().numpy().astype(np.float64)
    bad = (pos < 0) | (pos >= Lmax)
    assert np.isnan(got[bad]).all()
    ok = ~bad
    bound = 2.0 ** -8 * np.abs(want[ok]) + 2.0 ** -12 * np.abs(att.bf16_to_f64(v1)).max()
    assert (np.abs(got[ok] - want[ok]) <= bound).all()
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.abs(lg[ok] - want_lse[ok]).max() <= 2e-5
