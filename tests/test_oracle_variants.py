"""Pins of the oracle's normalisation variants ("Making Dr GRPO go brrr",
sections "GRPO" and "Dr. GRPO"): GRPO's group-standardised advantage,
GRPO's per-response mean (the length bias Dr. GRPO removes), and the token
mean the Dr. GRPO pseudo-code contrasts with its token sum.

Each variant is tied to hand-worked closed forms, an independent numpy
computation, invariants of its definition, the step-0 identity it implies,
central finite differences of the oracle's own loss, and the definition
written directly in PyTorch and differentiated by autograd."""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import ADV_CENTER, ADV_ZSCORE, AGG_SEQ_MEAN, AGG_TOKEN_MEAN, AGG_TOKEN_SUM


def _read_cases(path):
    with open(path) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- z-score advantage
def test_zscore_golden(golden_dir):
    """Hand-worked closed forms, to binary32 rounding (2 ulp)."""
    for line in _read_cases(os.path.join(golden_dir, "zscore_cases.txt")):
        g, rew, want = (p.strip() for p in line.split("|"))
        r = np.array([float(x) for x in rew.split()], dtype=np.float32)
        a = oracle.group_advantage(r, int(g), ADV_ZSCORE).astype(np.float64)
        w = np.array([float(x) for x in want.split()])
        assert np.all(np.abs(a - w) <= 2 * np.spacing(np.float32(np.abs(w).max() + 1))), line
        assert np.array_equal(a == 0, w == 0), line


def test_zscore_against_numpy_std():
    """Independent computation: numpy's mean and sample standard deviation
    (ddof=1) in binary64, on graded and Bernoulli rewards."""
    rng = np.random.default_rng(5)
    for G in (2, 4, 8, 16):
        r = rng.choice(np.array([0, 0.25, 0.5, 0.75, 1], np.float32), size=64 * G)
        r[:G] = 1.0  # a uniform group
        a = oracle.group_advantage(r, G, ADV_ZSCORE).astype(np.float64).reshape(-1, G)
        rg = r.astype(np.float64).reshape(-1, G)
        sd = rg.std(axis=1, ddof=1, keepdims=True)
        same = (rg == rg[:, :1]).all(axis=1)
        want = np.where(same[:, None], 0.0, (rg - rg.mean(axis=1, keepdims=True)) /
                        np.where(sd == 0, 1, sd))
        assert np.abs(a - want).max() <= 1e-6 * max(1.0, np.abs(want).max()), G


def test_zscore_invariants():
    """sum_j A_j = 0, sum_j A_j^2 = G - 1 (sample-std normalisation) and
    invariance under a positive affine change of the rewards."""
    cfg = synth.get_config("qwen_kl_b16g8c1024")
    case = synth.make_case(cfg)
    G = cfg.G
    a = oracle.group_advantage(case.rewards, G, ADV_ZSCORE).astype(np.float64).reshape(-1, G)
    live = (a != 0).any(axis=1)
    assert live.sum() >= 10
    assert np.abs(a[live].sum(axis=1)).max() < 1e-5
    assert np.abs((a[live] ** 2).sum(axis=1) - (G - 1)).max() < 1e-5
    b = oracle.group_advantage(3 * case.rewards + 0.5, G, ADV_ZSCORE).astype(np.float64)
    assert np.abs(b.reshape(-1, G) - a).max() < 1e-5
    # the centred (Dr. GRPO) advantage is the same vector before the division
    c = oracle.group_advantage(case.rewards, G, ADV_CENTER).astype(np.float64).reshape(-1, G)
    k = (c[live] * a[live]).sum(axis=1, keepdims=True) / (a[live] ** 2).sum(axis=1, keepdims=True)
    assert (k > 0).all()
    assert np.abs(c[live] - k * a[live]).max() <= 1e-6


def test_zscore_amplifies_low_variance_groups():
    """'Difficulty bias': the same single success gets a larger advantage in a
    group whose rewards vary less (1 of 8 correct vs 4 of 8 correct)."""
    easy = oracle.group_advantage(np.array([1, 0, 0, 0, 0, 0, 0, 0], np.float32), 8, ADV_ZSCORE)
    mid = oracle.group_advantage(np.array([1, 1, 1, 1, 0, 0, 0, 0], np.float32), 8, ADV_ZSCORE)
    assert easy[0] > 2 * mid[0]
    cen_e = oracle.group_advantage(np.array([1, 0, 0, 0, 0, 0, 0, 0], np.float32), 8)
    cen_m = oracle.group_advantage(np.array([1, 1, 1, 1, 0, 0, 0, 0], np.float32), 8)
    assert cen_e[0] > cen_m[0] and easy[0] / cen_e[0] > mid[0] / cen_m[0]


# ---------------------------------------------------------------- aggregation divisors
def test_row_divisor_definitions():
    lens = np.array([3, 1, 16, 5], np.int32)
    assert oracle.row_divisor(lens, 2.0, AGG_TOKEN_SUM).tolist() == [2.0] * 4
    assert oracle.row_divisor(lens, 2.0, AGG_SEQ_MEAN).tolist() == [6.0, 2.0, 32.0, 10.0]
    assert oracle.row_divisor(lens, 2.0, AGG_TOKEN_MEAN).tolist() == [50.0] * 4


def _tiny(adv_mode=ADV_CENTER):
    cfg = synth.get_config("tiny_fp32")
    case = synth.make_case(cfg)
    x = case.logits_rows_f32(np.arange(cfg.T)).astype(np.float64)
    _, logp, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    logp = logp.reshape(cfg.N, cfg.C)
    old = synth.perturb(logp, case.old_noise)
    lens = oracle.completion_len(case.tokens, cfg.eos_id)
    adv = oracle.group_advantage(case.rewards, cfg.G, adv_mode)
    return cfg, case, x, old, lens, adv


@pytest.mark.parametrize("adv_mode", [ADV_CENTER, ADV_ZSCORE])
def test_step0_identities(adv_mode):
    """At inner step 0 the ratio is 1 and lambda = -A_i per counted token, so
    token sum: L = -sum A_i |o_i| / kappa; per-response mean: L = -sum A_i /
    kappa; token mean: L = -sum A_i |o_i| / (kappa sum |o_i|)."""
    cfg, case, x, old, lens, adv = _tiny(adv_mode)
    logp = old.astype(np.float64)
    A = adv.astype(np.float64)
    k = cfg.norm_const
    want = {AGG_TOKEN_SUM: -math.fsum(A * lens) / k,
            AGG_SEQ_MEAN: -math.fsum(A) / k,
            AGG_TOKEN_MEAN: -math.fsum(A * lens) / (k * lens.sum())}
    scale = float(np.abs(A * lens).sum()) / k
    for agg, w in want.items():
        lam, coef, _ = oracle.token_terms(logp, old, None, adv, lens, cfg.eps, 0.0, k, agg)
        L = oracle.loss_sum(lam, k, lens, agg)
        assert abs(L - w) <= 1e-14 * scale, (agg, L, w)
    if adv_mode == ADV_CENTER:  # dyadic rewards: the per-response mean cancels exactly
        lam, _, _ = oracle.token_terms(logp, old, None, adv, lens, cfg.eps, 0.0, k, AGG_SEQ_MEAN)
        assert oracle.loss_sum(lam, k, lens, AGG_SEQ_MEAN) == 0.0


def test_length_bias_of_per_response_mean():
    """'Dr. GRPO', length bias: under the per-response mean a token's gradient
    coefficient is A_i / (kappa |o_i|) at ratio 1, so a longer wrong answer
    gets a weaker per-token penalty; the token sum gives every token A_i /
    kappa whatever the length."""
    cfg, case, x, old, lens, adv = _tiny()
    logp = old.astype(np.float64)
    k = cfg.norm_const
    mask = np.arange(cfg.C)[None, :] < lens[:, None]
    A = adv.astype(np.float64)[:, None] * np.ones((1, cfg.C))
    _, c_seq, _ = oracle.token_terms(logp, old, None, adv, lens, cfg.eps, 0.0, k, AGG_SEQ_MEAN)
    _, c_sum, _ = oracle.token_terms(logp, old, None, adv, lens, cfg.eps, 0.0, k, AGG_TOKEN_SUM)
    L = lens[:, None] * np.ones((1, cfg.C))
    assert np.array_equal(c_seq[mask], (A / (k * L))[mask])
    assert np.array_equal(c_sum[mask], (A / k)[mask])
    neg = np.flatnonzero(adv < 0)
    i_short, i_long = neg[np.argmin(lens[neg])], neg[np.argmax(lens[neg])]
    assert lens[i_long] > lens[i_short]
    assert abs(c_seq[i_long, 0]) < abs(c_seq[i_short, 0])


def _variant_loss(cfg, case, x, old, ref, beta, adv_mode, agg):
    return oracle.loss_fwd_bwd(x, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                               cfg.eps, beta, cfg.norm_const, adv_mode=adv_mode, agg=agg)


@pytest.mark.parametrize("adv_mode,agg", [(ADV_ZSCORE, AGG_SEQ_MEAN), (ADV_CENTER, AGG_TOKEN_MEAN),
                                          (ADV_ZSCORE, AGG_TOKEN_SUM)])
def test_variant_finite_differences(adv_mode, agg):
    """Central differences of each variant's loss equal its gradient on every
    logit of the tiny workload (with a KL term)."""
    cfg, case, x, old, lens, adv = _tiny(adv_mode)
    _, logp, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    ref = synth.perturb(logp.reshape(cfg.N, cfg.C), 2.0 * case.old_noise)
    beta = 0.04
    res = _variant_loss(cfg, case, x, old, ref, beta, adv_mode, agg)
    r = np.exp(res.logp - old.astype(np.float64))
    near = ((np.abs(r - (1 - cfg.eps)) < 1e-4) | (np.abs(r - (1 + cfg.eps)) < 1e-4)).reshape(-1)
    h = 1e-6
    rows = np.flatnonzero(~near)
    rng = np.random.default_rng(adv_mode * 3 + agg)
    rows = rng.choice(rows, 24, replace=False)
    fd = np.zeros((rows.size, cfg.V))
    for n, kk in enumerate(rows):
        for v in range(cfg.V):
            xp = x.copy()
            xp[kk, v] += h
            xm = x.copy()
            xm[kk, v] -= h
            fd[n, v] = (_variant_loss(cfg, case, xp, old, ref, beta, adv_mode, agg).loss -
                        _variant_loss(cfg, case, xm, old, ref, beta, adv_mode, agg).loss) / (2 * h)
    err = np.abs(fd - res.dlogits[rows]).max()
    assert err < 5e-8 * max(1.0, np.abs(res.dlogits).max() * cfg.norm_const), err
    assert np.abs(res.dlogits[rows]).max() > 0


@pytest.mark.parametrize("adv_mode,agg", [(ADV_ZSCORE, AGG_SEQ_MEAN), (ADV_CENTER, AGG_TOKEN_MEAN),
                                          (ADV_ZSCORE, AGG_TOKEN_SUM)])
def test_variant_against_autograd_of_the_definition(adv_mode, agg):
    """GRPO (std-normalised advantage, per-response mean) and the token mean
    written directly in PyTorch (float64, CPU) and differentiated by autograd."""
    import torch

    cfg = synth.get_config("clip_heavy_f32").with_(beta=0.04, ref_noise=0.2)
    case = synth.make_case(cfg)
    x = case.logits_rows_f32(np.arange(cfg.T)).astype(np.float64)
    _, logp, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    logp = logp.reshape(cfg.N, cfg.C)
    old = synth.perturb(logp, case.old_noise)
    ref = synth.perturb(logp, case.ref_noise)
    res = _variant_loss(cfg, case, x, old, ref, cfg.beta, adv_mode, agg)

    X = torch.tensor(x.reshape(cfg.N, cfg.C, cfg.V), requires_grad=True)
    tok = torch.tensor(case.tokens)
    lp = torch.log_softmax(X, dim=-1).gather(-1, tok[..., None])[..., 0]
    R = torch.tensor(case.rewards, dtype=torch.float64).view(cfg.B, cfg.G)
    A = R - R.mean(dim=1, keepdim=True)
    if adv_mode == ADV_ZSCORE:
        sd = R.std(dim=1, keepdim=True)  # torch's default: sample std
        A = torch.where(sd > 0, A / torch.where(sd > 0, sd, torch.ones_like(sd)), 0 * A)
    A = A.reshape(-1, 1)
    rho = torch.exp(lp - torch.tensor(old, dtype=torch.float64))
    surr = torch.minimum(rho * A, torch.clamp(rho, 1 - cfg.eps, 1 + cfg.eps) * A)
    d = torch.tensor(ref, dtype=torch.float64) - lp
    per_tok = -surr + cfg.beta * (torch.exp(d) - d - 1)
    is_eos = tok == cfg.eos_id
    first = torch.where(is_eos.any(1), is_eos.int().argmax(1), torch.full((cfg.N,), cfg.C - 1))
    m = (torch.arange(cfg.C)[None, :] <= first[:, None]).double()
    n_tok = m.sum(dim=1)

    def aggregate(t):
        if agg == AGG_SEQ_MEAN:
            return ((t * m).sum(dim=1) / n_tok).sum() / cfg.norm_const
        if agg == AGG_TOKEN_MEAN:
            return (t * m).sum() / (cfg.norm_const * n_tok.sum())
        return (t * m).sum() / cfg.norm_const

    L = aggregate(per_tok)
    L.backward()
    # the oracle forms the advantages in binary32 (relative rounding ~6e-8):
    # the loss agrees to 1e-6 of the same aggregation of |lambda|
    scale = float(aggregate(per_tok.detach().abs()))
    assert abs(L.item() - res.loss) <= 1e-6 * scale, (L.item(), res.loss, scale)
    g = X.grad.numpy().reshape(cfg.T, cfg.V)
    assert np.abs(g - res.dlogits).max() <= 1e-6 * np.abs(g).max()
