"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one step of the oracle to something other than the oracle
itself: values printed on the pages, hand-worked cases, closed forms,
invariants, brute force, central finite differences, or an independent
library implementation of the same textbook function.  A dropped term, a
wrong sign, index or branch anywhere in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

EPS = 0.2


def _read_cases(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line)
    return rows


# ---------------------------------------------------------------- completion mask
def test_mask_golden(golden_dir):
    """'Making Dr GRPO go brrr', 'The completion mask': first EOS inclusive;
    no EOS means every token counts."""
    for line in _read_cases(os.path.join(golden_dir, "mask_cases.txt")):
        eos, toks, want = (p.strip() for p in line.split("|"))
        tok = np.array([[int(x) for x in toks.split()]], dtype=np.int64)
        m = oracle.completion_mask(tok, int(eos))[0]
        assert m.tolist() == [int(x) for x in want.split()], line


def test_mask_brute_force_all_placements():
    """Every EOS/non-EOS pattern of rows up to C=10: the mask equals 'no EOS
    strictly before t' (a prefix-count characterisation, not the oracle's
    first-index loop)."""
    eos = 3
    for C in range(1, 11):
        pats = np.array([[(k >> t) & 1 for t in range(C)] for k in range(1 << C)])
        tok = np.where(pats == 1, eos, 7).astype(np.int64)
        m = oracle.completion_mask(tok, eos)
        eos_before = np.concatenate([np.zeros((len(pats), 1), int),
                                     np.cumsum(pats, axis=1)[:, :-1]], axis=1)
        want = (eos_before == 0).astype(np.uint8)
        assert np.array_equal(m, want), C
        # the mask is a prefix of ones, at least one long
        assert (m[:, 0] == 1).all()
        assert (np.diff(m.astype(int), axis=1) <= 0).all()


def test_mask_eos_outside_vocab_means_no_eos():
    tok = np.array([[1, 2, 3, 4]], dtype=np.int64)
    assert oracle.completion_len(tok, -1).tolist() == [4]


# ---------------------------------------------------------------- advantages
def test_advantage_golden(golden_dir):
    """'Making Dr GRPO go brrr', 'Dr. GRPO': A_i = R_i - group mean, no std."""
    for line in _read_cases(os.path.join(golden_dir, "advantage_cases.txt")):
        g, rew, want = (p.strip() for p in line.split("|"))
        r = np.array([float(x) for x in rew.split()], dtype=np.float32)
        a = oracle.group_advantage(r, int(g))
        w = np.array([float(x) for x in want.split()], dtype=np.float32)
        assert np.array_equal(a, w), line


def test_advantage_not_std_normalised():
    """GRPO's (R-mu)/sigma would give +-1 for {0,1,0,1}; Dr. GRPO keeps +-0.5."""
    a = oracle.group_advantage(np.array([0, 1, 0, 1], np.float32), 4)
    assert np.abs(a).max() == 0.5


def test_advantage_group_sums_and_layout():
    """Sum of advantages in a group is exactly 0 for dyadic rewards; groups are
    consecutive rows (rewards viewed as [B, G])."""
    cfg = synth.get_config("qwen_kl_b16g8c1024")
    case = synth.make_case(cfg)
    a = oracle.group_advantage(case.rewards, cfg.G).reshape(cfg.B, cfg.G)
    assert (a.astype(np.float64).sum(axis=1) == 0).all()
    r = case.rewards.reshape(cfg.B, cfg.G).astype(np.float64)
    assert np.array_equal(a.astype(np.float64), r - r.mean(axis=1, keepdims=True))


def test_uniform_groups_zero_advantage():
    """'The sparse-reward bottleneck': an all-zero or all-one group has zero
    centred advantages."""
    r = np.array([1, 1, 1, 1, 0, 0, 0, 0, 0, 1, 0, 0], np.float32)
    a = oracle.group_advantage(r, 4)
    assert (a[:8] == 0).all() and (a[8:] != 0).all()
    assert oracle.nocontrast_groups(r, 4) == 2


# ---------------------------------------------------------------- sparse-reward check
def test_sparse_reward_closed_forms_match_pages(golden_dir):
    for line in _read_cases(os.path.join(golden_dir, "sparse_reward.txt")):
        q, p, G, printed, dec = line.split()
        p, G, printed, dec = float(p), int(G), float(printed), int(dec)
        val = (1 - p) ** G if q == "all_fail" else (1 - p) ** G + p ** G
        assert round(val, dec) == printed, line


@pytest.mark.parametrize("p,G", [(0.05, 8), (0.05, 16), (0.2, 8)])
def test_bernoulli_no_contrast_frequency(p, G):
    """Empirical no-contrast frequency of the generator's Bernoulli rewards, as
    counted by the oracle, within 5 sigma of (1-p)^G + p^G over 10^6 groups."""
    M = 1_000_000
    u = synth.uniform01(424242 + G, synth.S_REWARDS, np.arange(M * G))
    r = (u < p).astype(np.float32)
    n = oracle.nocontrast_groups(r, G)
    q = (1 - p) ** G + p ** G
    sigma = math.sqrt(q * (1 - q) / M)
    assert abs(n / M - q) < 5 * sigma, (n / M, q)
    if (p, G) == (0.05, 8):
        assert round(n / M, 2) == 0.66  # the pages' "about two-thirds"


def test_dense_workload_has_every_row_active():
    """The dense-mode batch (no EOS, Bernoulli(0.5) rewards) leaves no token
    row inactive: every completion runs to C and every group has contrast."""
    cfg = synth.get_config("qwen_dense_b8g8c256")
    case = synth.make_case(cfg)
    assert (oracle.completion_len(case.tokens, cfg.eos_id) == cfg.C).all()
    assert (oracle.group_advantage(case.rewards, cfg.G) != 0).all()


# ---------------------------------------------------------------- log-probs
def test_logprob_normalises_and_is_nonpositive():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 3, size=(1, 257))
    V = x.shape[1]
    rows = np.repeat(x, V, axis=0)
    lse, logp, bad = oracle.row_logprob(rows, np.arange(V))
    assert bad == 0
    assert abs(np.exp(logp).sum() - 1.0) < 1e-12
    assert (logp <= 0).all()


def test_logprob_two_class_closed_form():
    a, b = 0.3, -1.7
    _, logp, _ = oracle.row_logprob(np.array([[a, b]]), np.array([0]))
    assert abs(logp[0] - (-math.log1p(math.exp(b - a)))) < 1e-15


def test_logprob_uniform_logits():
    V = 151936
    _, logp, _ = oracle.row_logprob(np.full((1, V), 2.5, np.float32), np.array([12345]))
    assert abs(logp[0] + math.log(V)) < 1e-12


def test_logprob_shift_against_full_sequence():
    """'Making Dr GRPO go brrr', 'compute_logprobs': logits at position t score
    token t+1, so the completion is scored by positions P-1 .. P+C-2 of the
    full prompt+completion sequence.  Passing that slice to the oracle must
    give, for token t, the log-softmax of full position P-1+t, computed here by
    scipy's log_softmax."""
    from scipy.special import log_softmax

    rng = np.random.default_rng(2)
    N, P, C, V = 3, 5, 6, 50
    full = rng.normal(0, 2, size=(N, P + C, V))
    comp = rng.integers(0, V, size=(N, C))
    sl = full[:, P - 1:P - 1 + C, :].reshape(N * C, V)
    _, logp, _ = oracle.row_logprob(sl, comp.reshape(-1))
    ls = log_softmax(full, axis=-1)
    want = np.array([[ls[i, P - 1 + t, comp[i, t]] for t in range(C)] for i in range(N)])
    assert np.allclose(logp.reshape(N, C), want, atol=1e-12, rtol=0)
    # the unshifted slice would be wrong
    wrong = np.array([[ls[i, P + t, comp[i, t]] for t in range(C - 1)] for i in range(N)])
    assert not np.allclose(logp.reshape(N, C)[:, :C - 1], wrong, atol=1e-3)


def test_logprob_bad_token_and_nan():
    x = np.zeros((2, 4))
    x[1, 2] = np.nan
    lse, logp, bad = oracle.row_logprob(x, np.array([4, 0]))
    assert bad == 1 and np.isnan(logp[0]) and np.isnan(logp[1]) and np.isnan(lse[1])


# ---------------------------------------------------------------- surrogate / KL
def test_clip_cases_golden(golden_dir):
    for line in _read_cases(os.path.join(golden_dir, "clip_cases.txt")):
        A, r, beta, lam_w, g_w = (float(x) for x in line.split())
        logp = np.array([[-2.0]])
        old = np.array([[-2.0 - math.log(r)]], dtype=np.float64)
        # old is fed as float32: re-derive the exact ratio the oracle sees
        old32 = old.astype(np.float32)
        ref = (np.array([[-2.0 + 0.1]])).astype(np.float32)
        lam, coef, _ = oracle.token_terms(logp, old32, ref if beta else None,
                                          np.array([A], np.float32), np.array([1], np.int32),
                                          EPS, beta, 1.0)
        assert abs(lam[0, 0] - lam_w) < 2e-6 * max(1, abs(lam_w)), line
        assert abs(-coef[0, 0] - g_w) < 2e-6 * max(1, abs(g_w)), line


def test_k3_closed_form_properties():
    d = np.linspace(-3, 3, 61)
    logp = np.full((1, d.size), -1.0)
    ref = (logp + d).astype(np.float32)
    dd = ref.astype(np.float64) - logp
    lam, coef, _ = oracle.token_terms(logp, logp.astype(np.float32), ref,
                                      np.array([0.0], np.float32),
                                      np.array([d.size], np.int32), EPS, 1.0, 1.0)
    k3 = lam[0]  # A = 0, beta = 1: lambda is the KL term alone
    assert (k3 >= 0).all()
    assert np.allclose(k3, np.exp(dd) - dd - 1, atol=1e-15)
    assert k3[30] == 0.0
    # derivative of k3 with respect to logp: 1 - e^d (coef = -g/kappa)
    assert np.allclose(-coef[0], 1 - np.exp(dd), atol=1e-15)


# ---------------------------------------------------------------- whole pass
def _tiny_f64(name="tiny_fp32", old_noise=None, beta=None, ref_noise=None):
    cfg = synth.get_config(name)
    if old_noise is not None:
        cfg = cfg.with_(old_noise=old_noise)
    if beta is not None:
        cfg = cfg.with_(beta=beta, ref_noise=ref_noise)
    case = synth.make_case(cfg)
    x = case.logits_rows_f32(np.arange(cfg.T)).astype(np.float64)
    _, logp, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    logp = logp.reshape(cfg.N, cfg.C)
    old = synth.perturb(logp, case.old_noise)
    ref = None if case.ref_noise is None else synth.perturb(logp, case.ref_noise)
    return cfg, case, x, old, ref


def _loss(cfg, case, x, old, ref, kappa=None):
    return oracle.loss_fwd_bwd(x, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                               cfg.eps, cfg.beta, kappa or cfg.norm_const, want_dlogits=True)


def test_step0_identity_exact():
    """'Making Dr GRPO go brrr', 'The loss': at inner step 0 current = old
    log-probs, the ratio is exactly 1 and the loss is -sum_i A_i |o_i| / kappa."""
    cfg, case, x, old, ref = _tiny_f64()
    logp = old.astype(np.float64)  # current log-probs equal to the stored old ones
    lens = oracle.completion_len(case.tokens, cfg.eos_id)
    adv = oracle.group_advantage(case.rewards, cfg.G)
    lam, coef, stats = oracle.token_terms(logp, old, None, adv, lens, cfg.eps, 0.0, cfg.norm_const)
    L = oracle.loss_sum(lam, cfg.norm_const)
    want = -float((adv.astype(np.float64) * lens).sum()) / cfg.norm_const
    assert L == want and L != 0.0
    assert stats.tolist() == [0, 0]


def test_step0_identity_through_logits():
    cfg, case, x, old, ref = _tiny_f64()
    lse, logp, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    res = oracle.loss_fwd_bwd(x, case.tokens, cfg.eos_id, case.rewards,
                              logp.reshape(cfg.N, cfg.C).astype(np.float32), None, cfg.G, cfg.eps,
                              0.0, cfg.norm_const)
    want = -float((res.adv.astype(np.float64) * res.len).sum()) / cfg.norm_const
    assert abs(res.loss - want) < 1e-6 * abs(want)


def test_uniform_group_zero_gradient_and_kl_exception():
    """Check (a): with beta = 0 an all-equal group contributes nothing; with a
    KL term its rows are no longer zero ('The sparse-reward bottleneck')."""
    cfg, case, x, old, ref = _tiny_f64()
    res = _loss(cfg, case, x, old, ref)
    G, C = cfg.G, cfg.C
    assert (case.rewards[:G] == case.rewards[0]).all()
    assert (res.lam[:G] == 0).all()
    assert (res.dlogits[:G * C] == 0).all()
    assert np.abs(res.dlogits[G * C:]).max() > 0
    ref2 = synth.perturb(res.logp, 0.1 * case.old_noise / 0.05)
    res2 = oracle.loss_fwd_bwd(x, case.tokens, cfg.eos_id, case.rewards, old, ref2, cfg.G,
                               cfg.eps, 0.04, cfg.norm_const)
    lens = res2.len[:G]
    rows = np.concatenate([np.arange(i * C, i * C + lens[i]) for i in range(G)])
    assert np.abs(res2.dlogits[rows]).min(axis=1).max() > 0
    assert (np.abs(res2.dlogits[rows]).max(axis=1) > 0).all()


def test_masked_tokens_are_exact_zero():
    cfg, case, x, old, ref = _tiny_f64()
    res = _loss(cfg, case, x, old, ref)
    mask = np.arange(cfg.C)[None, :] < res.len[:, None]
    assert (res.lam[~mask] == 0).all()
    assert (res.dlogits[(~mask).reshape(-1)] == 0).all()
    # whatever the logits hold at masked positions
    x2 = x.copy()
    x2[(~mask).reshape(-1)] = np.nan
    res2 = _loss(cfg, case, x2, old, ref)
    assert res2.loss == res.loss
    assert np.array_equal(res2.dlogits, res.dlogits)


def test_kappa_scaling():
    cfg, case, x, old, ref = _tiny_f64()
    r1 = _loss(cfg, case, x, old, ref, kappa=1.0)
    r3 = _loss(cfg, case, x, old, ref, kappa=3.0)
    assert abs(r1.loss - 3 * r3.loss) <= 1e-15 * abs(r1.loss)
    assert np.allclose(r1.dlogits, 3 * r3.dlogits, rtol=1e-14, atol=0)


def test_gradient_row_identities():
    cfg, case, x, old, ref = _tiny_f64()
    res = _loss(cfg, case, x, old, ref)
    D = res.dlogits
    tok = case.tokens.reshape(-1)
    coef = res.coef.reshape(-1)
    assert np.allclose(D.sum(axis=1), 0, atol=1e-16)
    p_y = np.exp(res.logp.reshape(-1))
    act = coef != 0
    assert np.allclose(D[act, tok[act]], coef[act] * (p_y[act] - 1), rtol=1e-12, atol=0)
    off = D[act].copy()
    off[np.arange(off.shape[0]), tok[act]] = 0
    assert ((off * np.sign(coef[act])[:, None]) >= 0).all()


def _fd_check(cfg, case, x, old, ref, h=1e-6, tol=2e-8):
    res = _loss(cfg, case, x, old, ref)
    r = np.exp(res.logp - old.astype(np.float64))
    near = (np.abs(r - (1 - cfg.eps)) < 1e-4) | (np.abs(r - (1 + cfg.eps)) < 1e-4)
    skip_rows = set(np.flatnonzero(near.reshape(-1)).tolist())
    fd = np.zeros_like(x)
    for k in range(x.shape[0]):
        if k in skip_rows:
            continue
        for v in range(x.shape[1]):
            xp = x.copy()
            xp[k, v] += h
            xm = x.copy()
            xm[k, v] -= h
            fd[k, v] = (_loss(cfg, case, xp, old, ref).loss
                        - _loss(cfg, case, xm, old, ref).loss) / (2 * h)
    keep = np.array([k not in skip_rows for k in range(x.shape[0])])
    err = np.abs(fd[keep] - res.dlogits[keep]).max()
    assert err < tol, err
    return res


def test_finite_differences_tiny():
    """Check (c): central differences of the oracle's own loss equal its
    gradient on every logit of the tiny workload."""
    cfg, case, x, old, ref = _tiny_f64()
    _fd_check(cfg, case, x, old, ref)


def test_finite_differences_clip_heavy_and_kl():
    """Central differences where the clip is active on both sides and a KL
    term is present."""
    cfg = synth.get_config("clip_heavy_f32").with_(C=6, beta=0.04, ref_noise=0.2)
    case = synth.make_case(cfg)
    x = case.logits_rows_f32(np.arange(cfg.T)).astype(np.float64)
    _, logp, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    logp = logp.reshape(cfg.N, cfg.C)
    old = synth.perturb(logp, case.old_noise)
    ref = synth.perturb(logp, case.ref_noise)
    res = _fd_check(cfg, case, x, old, ref, tol=5e-8)
    assert res.stats[1] > 0  # some tokens have their surrogate cut by the clip
    r = np.exp(res.logp - old.astype(np.float64))
    mask = np.arange(cfg.C)[None, :] < res.len[:, None]
    A = res.adv[:, None] * np.ones((1, cfg.C))
    assert ((r > 1 + cfg.eps) & (A > 0) & mask).any() and ((r < 1 - cfg.eps) & (A < 0) & mask).any()
    assert ((r > 1 + cfg.eps) & (A < 0) & mask).any() or ((r < 1 - cfg.eps) & (A > 0) & mask).any()


def test_against_autograd_of_the_definition():
    """The same loss written directly in PyTorch (float64, CPU), differentiated
    by autograd: loss and gradient agree with the oracle to 1e-12."""
    import torch

    cfg = synth.get_config("clip_heavy_f32").with_(beta=0.04, ref_noise=0.2)
    case = synth.make_case(cfg)
    x = case.logits_rows_f32(np.arange(cfg.T)).astype(np.float64)
    _, logp, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    logp = logp.reshape(cfg.N, cfg.C)
    old = synth.perturb(logp, case.old_noise)
    ref = synth.perturb(logp, case.ref_noise)
    res = oracle.loss_fwd_bwd(x, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                              cfg.eps, cfg.beta, cfg.norm_const)

    X = torch.tensor(x.reshape(cfg.N, cfg.C, cfg.V), requires_grad=True)
    tok = torch.tensor(case.tokens)
    lp = torch.log_softmax(X, dim=-1).gather(-1, tok[..., None])[..., 0]
    R = torch.tensor(case.rewards, dtype=torch.float64).view(cfg.B, cfg.G)
    A = (R - R.mean(dim=1, keepdim=True)).reshape(-1, 1)
    rho = torch.exp(lp - torch.tensor(old, dtype=torch.float64))
    surr = torch.minimum(rho * A, torch.clamp(rho, 1 - cfg.eps, 1 + cfg.eps) * A)
    d = torch.tensor(ref, dtype=torch.float64) - lp
    per_tok = -surr + cfg.beta * (torch.exp(d) - d - 1)
    is_eos = tok == cfg.eos_id
    first = torch.where(is_eos.any(1), is_eos.int().argmax(1), torch.full((cfg.N,), cfg.C - 1))
    m = (torch.arange(cfg.C)[None, :] <= first[:, None]).double()
    L = (per_tok * m).sum() / cfg.norm_const
    L.backward()
    assert abs(L.item() - res.loss) < 1e-12 * max(1.0, abs(res.loss))
    g = X.grad.numpy().reshape(cfg.T, cfg.V)
    assert np.abs(g - res.dlogits).max() < 1e-12
