"""Shared helpers of the parity tests: inputs from the seeded generators,
expected values from the oracle only."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import synth

F32_TOL = dict(loss_rel=1e-5, d_abs=1e-5, d_rel_max=1e-5, d_rel_elem=1e-5)
BF16_TOL = dict(loss_rel=2e-3, d_abs=4e-3, d_rel_max=1e-2, d_rel_elem=2.0 ** -7)
# A token whose oracle ratio lies this close to a clip boundary may take the
# other branch on the GPU (binary32 / bfloat16 inputs); its row is exempt.
TAU_R = {"f32": 5e-6, "bf16": 1e-4}


def tol(cfg):
    return F32_TOL if cfg.dtype == "f32" else BF16_TOL


def f32(v: float) -> float:
    """The binary32 value the GPU receives, widened for the oracle."""
    return float(np.float32(v))


@functools.lru_cache(maxsize=None)
def small_case(name: str, kappa: float | None = None):
    """(cfg, case, host logits, logp_old, logp_ref, oracle Result) for a case
    small enough to hold [T, V] in host memory."""
    cfg = synth.get_config(name)
    case = synth.make_case(cfg)
    x = case.logits_rows(np.arange(cfg.T))
    _, logp, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    logp = logp.reshape(cfg.N, cfg.C)
    old = synth.perturb(logp, case.old_noise)
    ref = None if case.ref_noise is None else synth.perturb(logp, case.ref_noise)
    k = cfg.norm_const if kappa is None else kappa
    res = oracle.loss_fwd_bwd(x, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                              f32(cfg.eps), f32(cfg.beta), f32(k))
    return cfg, case, x, old, ref, res


def oracle_logp_all(case, block_rows: int = 1024):
    """Oracle (lse, logp) of every token row, generating logits block by block
    on the host (never holding the whole [T, V] tensor)."""
    cfg = case.cfg
    T = cfg.T
    lse = np.empty(T)
    logp = np.empty(T)
    tok = case.tokens.reshape(-1)
    for r0 in range(0, T, block_rows):
        rows = np.arange(r0, min(T, r0 + block_rows))
        x = case.logits_rows(rows)
        l, p, _ = oracle.row_logprob(x, tok[rows])
        lse[rows] = l
        logp[rows] = p
    return lse.reshape(cfg.N, cfg.C), logp.reshape(cfg.N, cfg.C)


def to_device_logits(x: np.ndarray, cfg, device):
    import torch

    if cfg.dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return t.reshape(cfg.N, cfg.C, cfg.V).to(device)


def dlogits_to_f64(d) -> np.ndarray:
    return d.float().cpu().numpy().astype(np.float64).reshape(-1, d.shape[-1])


def exempt_rows(cfg, res, old) -> np.ndarray:
    """Token rows (flat indices) whose ratio sits on a clip boundary."""
    r = np.exp(res.logp - old.astype(np.float64))
    A = np.repeat(res.adv[:, None], cfg.C, axis=1)
    tau = TAU_R[cfg.dtype]
    e = f32(cfg.eps)
    near = ((np.abs(r - (1 - e)) <= tau) | (np.abs(r - (1 + e)) <= tau)) & (A != 0)
    mask = np.arange(cfg.C)[None, :] < res.len[:, None]
    return np.flatnonzero((near & mask).reshape(-1))


# absolute accuracy of a log-prob accumulated in binary32 from exact inputs
LOGP_ACC = 1e-6


def coef_condition(res, old, ref, eps: float, beta: float) -> np.ndarray:
    """Relative condition number of each token's gradient coefficient with
    respect to its log-prob, from the oracle's values: coef = -g/div with
    g = -A r chi + beta (1 - e^d), so |dg/dlogp| / |g| = (|A| r chi + beta
    e^d) / |g| (r = e^(logp - old), d = ref - logp).  Large where the
    surrogate and KL parts cancel or d ~ 0 in a KL-only gradient; 0 for
    tokens without gradient.  Flat [T]."""
    logp = res.logp
    A = res.adv.astype(np.float64)[:, None] * np.ones_like(logp)
    r = np.exp(logp - old.astype(np.float64))
    cut = ((A > 0) & (r > 1 + eps)) | ((A < 0) & (r < 1 - eps))
    chi = np.where(cut, 0.0, 1.0)
    ed = np.exp(ref.astype(np.float64) - logp) if ref is not None and beta else np.zeros_like(logp)
    g = -A * r * chi + beta * (1 - ed)
    with np.errstate(divide="ignore", invalid="ignore"):
        cond = (np.abs(A) * r * chi + beta * ed) / np.abs(g)
    return np.where(res.coef != 0, cond, 0.0).reshape(-1)


def compare_dlogits(cfg, got: np.ndarray, want: np.ndarray, rows=None, cond=None):
    """Assert the stated dlogits tolerances; returns (max abs err, max |ref|).
    `cond` (per row, from coef_condition) widens each row's element-wise
    relative bound by cond * LOGP_ACC: the coefficient is computed from a
    binary32 log-prob, so a row whose coefficient cancels carries that
    log-prob error amplified by its condition number."""
    t = tol(cfg)
    if rows is not None:
        got = got[rows]
        want = want[rows]
        if cond is not None:
            cond = cond[rows]
    err = np.abs(got - want)
    scale = float(np.abs(want).max()) if want.size else 0.0
    mx = float(err.max()) if err.size else 0.0
    assert mx <= t["d_abs"], f"dlogits max abs err {mx} > {t['d_abs']}"
    assert mx <= t["d_rel_max"] * scale + 1e-30, f"dlogits err {mx} > {t['d_rel_max']}*{scale}"
    rel = t["d_rel_elem"] if cond is None else t["d_rel_elem"] + LOGP_ACC * cond[:, None]
    bad = err > rel * np.abs(want) + 1e-30
    assert not bad.any(), (
        f"{int(bad.sum())} elements beyond {t['d_rel_elem']} relative; worst "
        f"got={got[bad][:4]} want={want[bad][:4]}")
    return mx, scale


def compare_loss(cfg, got: float, res):
    t = tol(cfg)
    ref = res.loss
    abs_scale = res.abs_sum / f32(cfg.norm_const) if res.abs_sum else 0.0
    cond = abs_scale / abs(ref) if ref != 0 else float("inf")
    if cond > 1e4:
        assert abs(got - ref) <= t["loss_rel"] * abs_scale, (got, ref, cond)
    else:
        assert abs(got - ref) <= t["loss_rel"] * abs(ref), (got, ref, abs(got - ref) / abs(ref))
    return cond


@functools.lru_cache(maxsize=None)
def lm_case(name: str):
    """(cfg, case, hidden bits [T,H], W bits [V,H], logp_old, logp_ref, oracle terms)
    for a fused lm_head case small enough for the oracle's full gradients."""
    from oracle import lmhead

    cfg = synth.get_config(name)
    case = synth.make_case(cfg)
    hb = case.hidden()
    Wb = case.weight()
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    _, logp = lmhead.token_rows(h64, W64, case.tokens.reshape(-1), np.arange(cfg.T))
    logp = logp.reshape(cfg.N, cfg.C)
    old = synth.perturb(logp, case.old_noise)
    ref = None if case.ref_noise is None else synth.perturb(logp, case.ref_noise)
    terms = lmhead.full(hb, Wb, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                        f32(cfg.eps), f32(cfg.beta), f32(cfg.norm_const))
    return cfg, case, hb, Wb, old, ref, terms


def scaled_bf16_rows(bits: np.ndarray, rows: np.ndarray, factor: float) -> np.ndarray:
    """bfloat16 bits with the given rows multiplied by a power of two (exact)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32).copy()
    f[rows] *= np.float32(factor)
    return (f.view(np.uint32) >> 16).astype(np.uint16)
