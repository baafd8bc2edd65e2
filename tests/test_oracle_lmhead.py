"""Pins of the fused lm_head oracle: it is the raw-logits oracle applied to
hidden . W^T, and its two weight gradients equal central finite differences
of its own loss."""
import numpy as np

import oracle
import synth
from oracle import lmhead
from _cases import f32


def _fd_case():
    cfg = synth.get_config("lmhead_fd")
    case = synth.make_case(cfg)
    h = lmhead.bf16_to_f64(case.hidden())
    W = lmhead.bf16_to_f64(case.weight())
    _, lp = lmhead.token_rows(h, W, case.tokens.reshape(-1), np.arange(cfg.T))
    lp = lp.reshape(cfg.N, cfg.C)
    old = synth.perturb(lp, case.old_noise)
    ref = synth.perturb(lp, case.ref_noise)
    return cfg, case, h, W, old, ref


def _loss(cfg, case, h, W, old, ref):
    return lmhead.loss_and_terms(h, W, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                                 cfg.eps, cfg.beta, cfg.norm_const)["loss"]


def test_lmhead_equals_raw_oracle_on_projected_logits():
    cfg, case, h, W, old, ref = _fd_case()
    t = lmhead.loss_and_terms(h, W, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                              cfg.eps, cfg.beta, cfg.norm_const)
    raw = oracle.loss_fwd_bwd(h @ W.T, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                              cfg.eps, cfg.beta, cfg.norm_const)
    assert abs(t["loss"] - raw.loss) <= 1e-13 * abs(raw.loss)
    assert t["loss"] != 0.0


def test_lmhead_gradients_by_finite_differences():
    """dL/dhidden = dlogits . W and dL/dW = dlogits^T . hidden, checked entry by
    entry against central differences (h = 1e-6) of the oracle's loss."""
    cfg, case, h, W, old, ref = _fd_case()
    t = lmhead.loss_and_terms(h, W, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                              cfg.eps, cfg.beta, cfg.norm_const)
    r = np.exp(t["logp"] - old.astype(np.float64))
    assert (np.abs(r - 1.2) > 1e-4).all() and (np.abs(r - 0.8) > 1e-4).all()
    logits = h @ W.T
    D = oracle.dlogits_rows(logits, case.tokens.reshape(-1), t["lse"], t["coef"])
    dh = D @ W
    dW = D.T @ h
    eps = 1e-6
    fd_h = np.zeros_like(h)
    for idx in np.ndindex(*h.shape):
        hp = h.copy(); hp[idx] += eps
        hm = h.copy(); hm[idx] -= eps
        fd_h[idx] = (_loss(cfg, case, hp, W, old, ref) - _loss(cfg, case, hm, W, old, ref)) / (2 * eps)
    assert np.abs(fd_h - dh).max() < 1e-8, np.abs(fd_h - dh).max()
    fd_W = np.zeros_like(W)
    for idx in np.ndindex(*W.shape):
        Wp = W.copy(); Wp[idx] += eps
        Wm = W.copy(); Wm[idx] -= eps
        fd_W[idx] = (_loss(cfg, case, h, Wp, old, ref) - _loss(cfg, case, h, Wm, old, ref)) / (2 * eps)
    assert np.abs(fd_W - dW).max() < 1e-8, np.abs(fd_W - dW).max()
    # the sampled-row helpers agree with the full products
    rows = t["active_rows"][:5]
    assert np.allclose(lmhead.dhidden_rows(h, W, case.tokens.reshape(-1), t, rows), dh[rows],
                       rtol=1e-12, atol=1e-15)
    vs = [0, 7, int(case.tokens.reshape(-1)[rows[0]]), cfg.V - 1]
    assert np.allclose(lmhead.dW_rows(h, W, case.tokens.reshape(-1), t, vs), dW[vs], rtol=1e-10,
                       atol=1e-14)
