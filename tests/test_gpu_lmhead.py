"""GPU parity of the fused lm_head variant against the CPU oracle.

Small cases: loss, every dhidden and dW entry.  Full size (B=8, G=8, C=512,
H=896, V=151936): loss over every token, sampled dhidden rows and dW rows.
Tolerances: loss rel <= 2e-3; dhidden and dW through ``_lmcheck``: every
element against a worst-case rounding model of the precision path (bfloat16
dlogits entering binary32 products, bfloat16 results), every row and part
against its RMS model, and the regression slope of each part, with the
vocabulary rows of dW that no active token sampled and the softmax part of
dhidden checked as parts of their own (test_lmcheck.py shows the checks fail
when one of those parts is wrong)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import rl_post_loss_dr_amd as dr
from oracle import lmhead
from _cases import f32, lm_case, scaled_bf16_rows
from _lmcheck import check_dW, check_dhidden

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bits_to_dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _dev_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run(cfg, case, hb, Wb, old, ref):
    loss, dh, dW = dr.lmhead_loss_fwd_bwd(
        _bits_to_dev(hb), _bits_to_dev(Wb), torch.from_numpy(case.tokens).to(DEV), cfg.eos_id,
        torch.from_numpy(case.rewards).to(DEV), torch.from_numpy(old).to(DEV),
        None if ref is None else torch.from_numpy(ref).to(DEV), G=cfg.G, eps=cfg.eps,
        beta=cfg.beta, norm_const=cfg.norm_const)
    torch.cuda.synchronize()
    return float(loss.item()), dh, dW


def check_small_grads(cfg, case, hb, Wb, t, dh, dW):
    """Every dhidden row and every dW row of a small case through the checker."""
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    tok = case.tokens.reshape(-1)
    D = t["dlogits"]
    act = t["active_rows"]
    r1 = check_dhidden(_dev_to_f64(dh), D, W64, t["coef"], tok)
    r2 = check_dW(_dev_to_f64(dW), D[act], h64[act], np.isin(np.arange(cfg.V), tok[act]))
    print(f"[{cfg.name}] {r1} {r2}", flush=True)


@pytest.mark.parametrize("name", ["lmhead_mini", "lmhead_multi", "lmhead_chunks3",
                                  "lmhead_wide_h", "lmhead_h1536"])
def test_lmhead_small(name):
    print(f"case {name}", flush=True)
    cfg, case, hb, Wb, old, ref, t = lm_case(name)
    loss, dh, dW = _run(cfg, case, hb, Wb, old, ref)
    assert abs(loss - t["loss"]) <= 2e-3 * abs(t["loss"]), (loss, t["loss"])
    check_small_grads(cfg, case, hb, Wb, t, dh, dW)
    # tokens without gradient have exactly zero dhidden rows
    zero = t["coef"] == 0
    assert (_dev_to_f64(dh)[zero] == 0).all()


def test_lmhead_deterministic():
    cfg, case, hb, Wb, old, ref, t = lm_case("lmhead_multi")
    l1, dh1, dW1 = _run(cfg, case, hb, Wb, old, ref)
    l2, dh2, dW2 = _run(cfg, case, hb, Wb, old, ref)
    assert l1 == l2 and torch.equal(dh1, dh2) and torch.equal(dW1, dW2)


def test_lmhead_rows_far_above_their_reference():
    """The forward product keeps exp(x - r) with r the sampled token's logit;
    rows whose largest logit lies more than 48 above it (here: every other
    token's hidden row scaled by 32, logits up to ~170: the first pass even
    overflows binary32 for some) make the
    call run the forward product again with those rows' maxima.  Loss and
    every gradient entry still match the oracle, and the result is the same
    on a second call."""
    cfg, case, _, Wb, _, _, _ = lm_case("lmhead_multi")
    hb = scaled_bf16_rows(case.hidden(), np.arange(0, cfg.T, 2), 32.0)
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    tok = case.tokens.reshape(-1)
    x = h64 @ W64.T
    gap = x.max(axis=1) - x[np.arange(cfg.T), tok]
    _, logp = lmhead.token_rows(h64, W64, tok, np.arange(cfg.T))
    logp = logp.reshape(cfg.N, cfg.C)
    old = synth.perturb(logp, case.old_noise)
    ref = synth.perturb(logp, case.ref_noise)
    t = lmhead.full(hb, Wb, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                    f32(cfg.eps), f32(cfg.beta), f32(cfg.norm_const))
    act = t["active_rows"]
    far = act[gap[act] > 48.0]
    print(f"{far.size} of {act.size} active rows beyond the window (max gap {gap[act].max():.1f})",
          flush=True)
    assert far.size >= 4 and far.size < act.size
    loss, dh, dW = _run(cfg, case, hb, Wb, old, ref)
    assert abs(loss - t["loss"]) <= 2e-3 * abs(t["loss"]), (loss, t["loss"])
    check_small_grads(cfg, case, hb, Wb, t, dh, dW)
    l2, dh2, dW2 = _run(cfg, case, hb, Wb, old, ref)
    assert l2 == loss and torch.equal(dh, dh2) and torch.equal(dW, dW2)


def test_lmhead_no_active_tokens():
    """All groups uniform and beta = 0: zero loss, zero gradients."""
    cfg, case, hb, Wb, old, ref, t = lm_case("lmhead_mini")
    rewards = np.ones_like(case.rewards)
    loss, dh, dW = dr.lmhead_loss_fwd_bwd(
        _bits_to_dev(hb), _bits_to_dev(Wb), torch.from_numpy(case.tokens).to(DEV), cfg.eos_id,
        torch.from_numpy(rewards).to(DEV), torch.from_numpy(old).to(DEV), None, G=cfg.G)
    torch.cuda.synchronize()
    assert float(loss.item()) == 0.0
    assert float(dh.float().abs().max()) == 0.0 and float(dW.float().abs().max()) == 0.0


def test_lmhead_full_size_sampled():
    cfg = synth.get_config("lmhead_b8g8c512")
    case = synth.make_case(cfg)
    print(f"[{cfg.name}] host inputs", flush=True)
    hb = case.hidden()
    Wb = case.weight()
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    lens = oracle.completion_len(case.tokens, cfg.eos_id)
    adv = oracle.group_advantage(case.rewards, cfg.G)
    mask = np.arange(cfg.C)[None, :] < lens[:, None]
    active = np.flatnonzero((mask & (adv[:, None] != 0)).reshape(-1))
    # logp_old only matters at active tokens; elsewhere any finite value
    print(f"[{cfg.name}] oracle log-probs of {active.size} active tokens", flush=True)
    _, lp_act = lmhead.token_rows(h64, W64, case.tokens.reshape(-1), active)
    lp = np.zeros(cfg.T)
    lp[active] = lp_act
    old = synth.perturb(lp.reshape(cfg.N, cfg.C), case.old_noise)
    t = lmhead.loss_and_terms(h64, W64, case.tokens, cfg.eos_id, case.rewards, old, None, cfg.G,
                              f32(cfg.eps), f32(cfg.beta), f32(cfg.norm_const))
    print(f"[{cfg.name}] device run", flush=True)
    loss, dh, dW = _run(cfg, case, hb, Wb, old, None)
    print(f"[{cfg.name}] loss gpu {loss!r} oracle {t['loss']!r}", flush=True)
    assert abs(loss - t["loss"]) <= 2e-3 * abs(t["loss"])
    rng = np.random.default_rng(cfg.seed)
    tok = case.tokens.reshape(-1)
    rows = np.unique(np.concatenate([rng.choice(active, 60, replace=False), active[:2],
                                     active[-2:], [0]]))
    print(f"[{cfg.name}] oracle dlogits of {rows.size} token rows", flush=True)
    D = lmhead.dlogits_token_rows(h64, W64, tok, t, rows)
    r1 = check_dhidden(_dev_to_f64(dh[torch.from_numpy(rows).to(DEV)]), D, W64, t["coef"][rows],
                       tok[rows])
    # vocabulary rows: some that active tokens sampled, more that none did
    # (their gradient is the softmax part alone), and both ends
    samp_ids = np.unique(tok[active])
    others = np.setdiff1d(np.arange(cfg.V), samp_ids)
    vs = np.unique(np.concatenate([rng.choice(samp_ids, 24, replace=False),
                                   rng.choice(others, 48, replace=False), [0, cfg.V - 1]]))
    print(f"[{cfg.name}] oracle dlogits columns of {vs.size} vocabulary rows", flush=True)
    Dc = lmhead.dlogits_vocab_cols(h64, W64, tok, t, vs)
    r2 = check_dW(_dev_to_f64(dW[torch.from_numpy(vs).to(DEV)]), Dc, h64[active],
                  np.isin(vs, samp_ids))
    print(f"[{cfg.name}] {r1} {r2}", flush=True)
    # every inactive token's dhidden row is exactly zero
    inactive = np.setdiff1d(np.arange(cfg.T), active)
    assert float(dh[torch.from_numpy(inactive).to(DEV)].float().abs().max()) == 0.0


def _logp_bound(h64, W64, rows):
    """Tolerance of a log-prob from binary32 MFMA logits: each logit's
    accumulation error is at most gamma_H * sum_k |h_k||w_k| (gamma_H =
    H u / (1 - H u), u = 2^-24), and log_softmax moves by at most twice the
    largest logit error; 1e-5 covers the binary32 exp / sum over V."""
    H = h64.shape[1]
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    a = np.abs(h64[rows]) @ np.abs(W64).T
    return 2 * gamma * a.max(axis=1) + 1e-5


@pytest.mark.parametrize("name", ["lmhead_mini", "lmhead_multi", "lmhead_chunks3",
                                  "lmhead_wide_h", "lmhead_h1536"])
def test_lmhead_logprobs_small(name):
    """Forward-only fused log-probs: every counted token against the oracle,
    zeros after the first EOS, and every token when no EOS id is given."""
    print(f"case {name}", flush=True)
    cfg, case, hb, Wb, old, ref, t = lm_case(name)
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    tok = case.tokens.reshape(-1)
    _, want = lmhead.token_rows(h64, W64, tok, np.arange(cfg.T))
    bound = _logp_bound(h64, W64, np.arange(cfg.T))
    hd, Wd, td = _bits_to_dev(hb), _bits_to_dev(Wb), torch.from_numpy(case.tokens).to(DEV)
    got = dr.lmhead_logprobs(hd, Wd, td, cfg.eos_id).cpu().numpy().astype(np.float64).reshape(-1)
    lens = oracle.completion_len(case.tokens, cfg.eos_id)
    counted = (np.arange(cfg.C)[None, :] < lens[:, None]).reshape(-1)
    assert (np.abs(got - want)[counted] <= bound[counted]).all(), float(
        np.abs(got - want)[counted].max())
    assert (got[~counted] == 0.0).all()
    got_all = dr.lmhead_logprobs(hd, Wd, td, -1).cpu().numpy().astype(np.float64).reshape(-1)
    assert (np.abs(got_all - want) <= bound).all()
    # the counted tokens are the same computation either way
    assert np.array_equal(got_all[counted], got[counted])


def test_lmhead_logprobs_rows_far_above_their_reference():
    """The forward-only pass sums exp(x - r) with r the sampled token's logit;
    rows whose largest logit lies more than 48 above it (every other token's
    hidden row scaled by 32) make the call redo every tile relative to the
    rows' maxima; every counted log-prob still matches the oracle, with and
    without an EOS id."""
    cfg, case, _, Wb, _, _, _ = lm_case("lmhead_multi")
    hb = scaled_bf16_rows(case.hidden(), np.arange(0, cfg.T, 2), 32.0)
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    tok = case.tokens.reshape(-1)
    x = h64 @ W64.T
    gap = x.max(axis=1) - x[np.arange(cfg.T), tok]
    lens = oracle.completion_len(case.tokens, cfg.eos_id)
    counted = (np.arange(cfg.C)[None, :] < lens[:, None]).reshape(-1)
    assert (gap[counted] > 48.0).sum() >= 4
    _, want = lmhead.token_rows(h64, W64, tok, np.arange(cfg.T))
    bound = _logp_bound(h64, W64, np.arange(cfg.T))
    hd, Wd, td = _bits_to_dev(hb), _bits_to_dev(Wb), torch.from_numpy(case.tokens).to(DEV)
    got = dr.lmhead_logprobs(hd, Wd, td, cfg.eos_id).cpu().numpy().astype(np.float64).reshape(-1)
    err = np.abs(got - want)
    assert (err[counted] <= bound[counted]).all(), float(err[counted].max())
    assert (got[~counted] == 0.0).all()
    got_all = dr.lmhead_logprobs(hd, Wd, td, -1).cpu().numpy().astype(np.float64).reshape(-1)
    assert (np.abs(got_all - want) <= bound).all()


def test_lmhead_logprobs_bad_token_is_nan():
    cfg, case, hb, Wb, old, ref, t = lm_case("lmhead_mini")
    tokens = case.tokens.copy()
    tokens[1, 0] = cfg.V + 5  # counted: no EOS id is given below
    got = dr.lmhead_logprobs(_bits_to_dev(hb), _bits_to_dev(Wb), torch.from_numpy(tokens).to(DEV),
                             -1).cpu().numpy()
    assert np.isnan(got[1, 0])
    assert np.isfinite(np.delete(got.reshape(-1), cfg.C)).all()


def test_lmhead_logprobs_full_size_sampled():
    """Full Qwen2.5-0.5B-shaped lm_head (T = 32,768 rows, V = 151,936, H = 896):
    sampled counted rows against the oracle, zeros after each first EOS."""
    cfg = synth.get_config("lmhead_b8g8c512")
    case = synth.make_case(cfg)
    print(f"[{cfg.name}] host inputs", flush=True)
    hb = case.hidden()
    Wb = case.weight()
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    lens = oracle.completion_len(case.tokens, cfg.eos_id)
    counted = (np.arange(cfg.C)[None, :] < lens[:, None]).reshape(-1)
    print(f"[{cfg.name}] device run", flush=True)
    got = dr.lmhead_logprobs(_bits_to_dev(hb), _bits_to_dev(Wb),
                             torch.from_numpy(case.tokens).to(DEV), cfg.eos_id)
    got = got.cpu().numpy().astype(np.float64).reshape(-1)
    assert (got[~counted] == 0.0).all()
    rng = np.random.default_rng(cfg.seed + 1)
    idx = np.flatnonzero(counted)
    rows = np.unique(np.concatenate([rng.choice(idx, 24, replace=False), idx[:2], idx[-2:]]))
    print(f"[{cfg.name}] oracle log-probs of {rows.size} sampled rows", flush=True)
    _, want = lmhead.token_rows(h64, W64, case.tokens.reshape(-1), rows)
    bound = _logp_bound(h64, W64, rows)
    err = np.abs(got[rows] - want)
    print(f"[{cfg.name}] max |logp err| {err.max():.3g} (bound min {bound.min():.3g})", flush=True)
    assert (err <= bound).all()
    assert np.isfinite(got[counted]).all()


def test_lmhead_bad_token_poisons_only_its_row():
    """A counted token id outside [0, V) in a row with gradient: the loss is
    NaN and the device status reports it; that token's dhidden row is NaN and
    its dlogits row takes no part in the products, so every other dhidden row
    and all of dW equal the oracle's gradients with that row removed."""
    cfg, case, hb, Wb, old, ref, t = lm_case("lmhead_mini")
    tok = case.tokens.copy()
    coef = t["coef"].reshape(cfg.N, cfg.C)
    i, tt = [(i, tt) for i in range(cfg.N) for tt in range(cfg.C)
             if coef[i, tt] != 0 and tok[i, tt] != cfg.eos_id][3]
    tok[i, tt] = cfg.V + 7
    pos = i * cfg.C + tt
    ws = torch.empty(dr.lmhead_workspace_bytes(cfg.N, cfg.C, cfg.V, cfg.H, cfg.G),
                     dtype=torch.uint8, device=DEV)
    loss, dh, dW = dr.lmhead_loss_fwd_bwd(
        _bits_to_dev(hb), _bits_to_dev(Wb), torch.from_numpy(tok).to(DEV), cfg.eos_id,
        torch.from_numpy(case.rewards).to(DEV), torch.from_numpy(old).to(DEV),
        None if ref is None else torch.from_numpy(ref).to(DEV), G=cfg.G, eps=cfg.eps,
        beta=cfg.beta, norm_const=cfg.norm_const, workspace=ws)
    torch.cuda.synchronize()
    assert np.isnan(float(loss.item()))
    assert dr.device_status(ws) == dr.ERR_TOKEN_RANGE
    got_h = _dev_to_f64(dh)
    assert np.isnan(got_h[pos]).all()
    keep = np.setdiff1d(np.arange(cfg.T), [pos])
    D = t["dlogits"].copy()
    D[pos] = 0.0
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    flat = case.tokens.reshape(-1)
    check_dhidden(got_h[keep], D[keep], W64, t["coef"][keep], flat[keep])
    act = np.setdiff1d(t["active_rows"], [pos])
    check_dW(_dev_to_f64(dW), D[act], h64[act], np.isin(np.arange(cfg.V), flat[act]))
