"""GPU parity on the degenerate cases of the method, against the oracle:
one completion per group (G = 1), a one-entry vocabulary (V = 1), one-token
completions (C = 1), every completion ending at t = 0, a batch with no reward
contrast, very large logits, and vocabulary entries at -inf.  Inputs are
seeded (numpy's generator); expected values come from the oracle only."""
import numpy as np
import pytest
import torch

import oracle
import rl_post_loss_dr_amd as dr
from _cases import coef_condition, compare_dlogits, f32

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


class _Cfg:
    def __init__(self, dtype, norm_const, eps=0.2, beta=0.0):
        self.dtype, self.norm_const, self.eps, self.beta = dtype, norm_const, eps, beta


def _bf16_bits(x):
    """Round binary64 values to bfloat16 (nearest even) and return the bits."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def _run_case(x, tokens, eos_id, rewards, G, dtype, beta=0.0, kappa=None, ref_noise=0.1,
              seed=0):
    """x: [N, C, V] binary64 logits (rounded to the dtype first)."""
    rng = np.random.default_rng(seed)
    N, C, V = x.shape
    if dtype == "bf16":
        xb = _bf16_bits(x.reshape(N * C, V))
        host = xb
        dev = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).reshape(N, C, V).to(DEV)
    else:
        host = x.reshape(N * C, V).astype(np.float32)
        dev = torch.from_numpy(host).reshape(N, C, V).to(DEV)
    _, logp, _ = oracle.row_logprob(host, tokens.reshape(-1))
    logp = np.nan_to_num(logp.reshape(N, C), nan=0.0)
    old = (logp + rng.normal(0, 0.05, logp.shape)).astype(np.float32)
    ref = (logp + rng.normal(0, ref_noise, logp.shape)).astype(np.float32) if beta else None
    kappa = float(G * C) if kappa is None else kappa
    res = oracle.loss_fwd_bwd(host, tokens, eos_id, rewards, old, ref, G, f32(0.2), f32(beta),
                              f32(kappa))
    aux = {"counts": torch.empty(2, dtype=torch.int64, device=DEV)}
    loss, d = dr.loss_fwd_bwd(dev, torch.from_numpy(tokens).to(DEV), eos_id,
                              torch.from_numpy(rewards).to(DEV), torch.from_numpy(old).to(DEV),
                              None if ref is None else torch.from_numpy(ref).to(DEV), G=G,
                              eps=0.2, beta=beta, norm_const=kappa, aux=aux,
                              out_counts=aux["counts"])
    torch.cuda.synchronize()
    got = d.float().cpu().numpy().astype(np.float64).reshape(N * C, V)
    cfg = _Cfg(dtype, kappa, beta=beta)
    cfg.cond = coef_condition(res, old, ref, f32(0.2), f32(beta))
    return float(loss.item()), got, res, aux, cfg


def _check(loss, got, res, aux, cfg):
    assert np.array_equal(aux["len"].cpu().numpy(), res.len)
    assert np.array_equal(aux["adv"].cpu().numpy().view(np.uint32), res.adv.view(np.uint32))
    rtol = 1e-5 if cfg.dtype == "f32" else 2e-3
    scale = res.abs_sum / cfg.norm_const
    assert abs(loss - res.loss) <= rtol * max(abs(res.loss), scale * 1e-4) + 1e-30, \
        (loss, res.loss)
    if np.abs(res.dlogits).max() > 0:
        compare_dlogits(cfg, got, res.dlogits, cond=cfg.cond)
    assert (got[res.coef.reshape(-1) == 0] == 0).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_completion_per_group(dtype):
    """G = 1: every group is uniform, so A = 0 everywhere; beta = 0 gives an
    exactly zero loss and gradient, beta > 0 the KL term alone."""
    rng = np.random.default_rng(1)
    N, C, V = 5, 6, 72
    x = rng.normal(0, 2, (N, C, V))
    tokens = rng.integers(1, V, (N, C)).astype(np.int64)
    tokens[1, 2] = 0
    rewards = rng.choice([0.0, 1.0], N).astype(np.float32)
    loss, got, res, aux, cfg = _run_case(x, tokens, 0, rewards, 1, dtype)
    assert loss == 0.0 and (got == 0).all() and (res.adv == 0).all()
    loss, got, res, aux, cfg = _run_case(x, tokens, 0, rewards, 1, dtype, beta=0.04)
    assert res.loss != 0.0
    _check(loss, got, res, aux, cfg)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_entry_vocabulary(dtype):
    """V = 1: the softmax is 1, every log-prob is 0 and the gradient vanishes."""
    rng = np.random.default_rng(2)
    N, C, V = 4, 5, 1
    x = rng.normal(0, 3, (N, C, V))
    tokens = np.zeros((N, C), np.int64)
    rewards = np.array([1, 0, 0, 1], np.float32)
    loss, got, res, aux, cfg = _run_case(x, tokens, -1, rewards, 2, dtype)
    assert (got == 0).all()
    assert (aux["len"].cpu().numpy() == C).all()
    _check(loss, got, res, aux, cfg)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_token_completions_and_eos_at_zero(dtype):
    """C = 1, and a batch in which every completion is its EOS at t = 0."""
    rng = np.random.default_rng(3)
    N, V = 8, 136
    x = rng.normal(0, 2, (N, 1, V))
    tokens = rng.integers(0, V, (N, 1)).astype(np.int64)
    rewards = np.array([1, 0, 0, 0, 1, 1, 0, 1], np.float32)
    _check(*_run_case(x, tokens, 7, rewards, 4, dtype))
    C = 9
    x = rng.normal(0, 2, (N, C, V))
    tokens = rng.integers(0, V, (N, C)).astype(np.int64)
    tokens[:, 0] = 7
    loss, got, res, aux, cfg = _run_case(x, tokens, 7, rewards, 4, dtype)
    assert (res.len == 1).all()
    _check(loss, got, res, aux, cfg)
    assert (got.reshape(N, C, V)[:, 1:] == 0).all()


def test_no_reward_contrast_anywhere():
    """Every group uniform ('The sparse-reward bottleneck'): zero loss, zero
    gradient, and the counter reports every group."""
    rng = np.random.default_rng(4)
    N, C, V = 16, 4, 96
    x = rng.normal(0, 2, (N, C, V))
    tokens = rng.integers(1, V, (N, C)).astype(np.int64)
    rewards = np.repeat(np.array([0, 1, 0, 0], np.float32), 4)
    loss, got, res, aux, cfg = _run_case(x, tokens, 0, rewards, 4, "bf16")
    assert loss == 0.0 and (got == 0).all()
    st = aux["stats"].cpu().numpy()
    assert st[0] == 4 and int(aux["counts"][1]) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_large_logits_and_masked_vocabulary(dtype):
    """Logits of magnitude ~1e3 (the online max keeps exp in range) and
    vocabulary entries at -inf (probability exactly 0, gradient exactly 0)."""
    rng = np.random.default_rng(5)
    N, C, V = 4, 6, 4104
    x = rng.normal(0, 300, (N, C, V))
    x[:, :, 1000:1400] = -np.inf
    tokens = rng.integers(0, 1000, (N, C)).astype(np.int64)
    rewards = np.array([1, 0, 0.5, 0.25], np.float32)
    loss, got, res, aux, cfg = _run_case(x, tokens, -1, rewards, 4, dtype, beta=0.04)
    assert np.isfinite(loss)
    _check(loss, got, res, aux, cfg)
    assert (got[:, 1000:1400] == 0).all()
