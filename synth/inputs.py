"""Assemble the small per-row / per-token synthetic arrays of a workload.

Nothing here computes any part of the loss: the arrays are token ids, EOS
placement, rewards and the noise that turns a log-prob into an "old" or
"reference" log-prob.  The log-prob itself is supplied by the caller.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import (S_EOS_POS, S_EOS_ROWS, S_OLD_NOISE, S_REF_NOISE, S_REWARDS, S_TOKENS,
               S_LOGITS, S_HIDDEN, S_WEIGHT, F32, BF16, draws, key, normal64, randint,
               uniform01, cpu_normal, cpu_normal_rows, bf16_bits_to_f32)
from .configs import Config


@dataclass
class Case:
    cfg: Config
    tokens: np.ndarray          # int64 [N, C]
    rewards: np.ndarray         # float32 [N]
    old_noise: np.ndarray       # float64 [N, C]
    ref_noise: np.ndarray | None  # float64 [N, C]

    @property
    def dtype_code(self) -> int:
        return F32 if self.cfg.dtype == "f32" else BF16

    # ---- logits (row r of the [N*C, V] tensor scores tokens.flat[r])
    def logits_rows(self, rows) -> np.ndarray:
        """Raw generated logits rows: float32 or bfloat16 bits (uint16)."""
        c = self.cfg
        return cpu_normal_rows(c.seed, S_LOGITS, rows, c.V, c.logit_std, self.dtype_code)

    def logits_all(self) -> np.ndarray:
        c = self.cfg
        return cpu_normal(c.seed, S_LOGITS, 0, c.T * c.V, c.logit_std,
                          self.dtype_code).reshape(c.T, c.V)

    def logits_rows_f32(self, rows) -> np.ndarray:
        raw = self.logits_rows(rows)
        return raw if self.cfg.dtype == "f32" else bf16_bits_to_f32(raw)

    # ---- fused lm_head inputs
    def hidden(self) -> np.ndarray:
        c = self.cfg
        return cpu_normal(c.seed, S_HIDDEN, 0, c.T * c.H, c.hidden_std, BF16).reshape(c.T, c.H)

    def weight(self) -> np.ndarray:
        c = self.cfg
        return cpu_normal(c.seed, S_WEIGHT, 0, c.V * c.H, c.w_std, BF16).reshape(c.V, c.H)


def _tokens(cfg: Config) -> np.ndarray:
    N, C = cfg.N, cfg.C
    allowed = cfg.tok_hi - cfg.tok_lo
    eos_in = cfg.tok_lo <= cfg.eos_id < cfg.tok_hi
    n = allowed - (1 if eos_in else 0)
    raw = randint(cfg.seed, S_TOKENS, np.arange(N * C), n) + cfg.tok_lo
    if eos_in:
        raw = np.where(raw >= cfg.eos_id, raw + 1, raw)
    tok = raw.reshape(N, C).astype(np.int64)
    if cfg.eos_rows <= 0:
        return tok
    order = np.argsort(draws(key(cfg.seed, S_EOS_ROWS), np.arange(N)), kind="stable")
    rows = order[: cfg.eos_rows]
    pos = randint(cfg.seed, S_EOS_POS, rows, C)
    for j, r in enumerate(rows):
        if j < cfg.eos_t0_rows:
            t = 0
        elif cfg.eos_t0_rows > 0:
            t = 1 + int(randint(cfg.seed, S_EOS_POS, [N + r], C - 1)[0])
        else:
            t = int(pos[j])
        tok[r, t] = cfg.eos_id
        if cfg.eos_pad:
            tok[r, t:] = cfg.eos_id
        if cfg.extra_eos and t + 1 < C:
            t2 = t + 1 + int(randint(cfg.seed, S_EOS_POS, [2 * N + r], C - t - 1)[0])
            tok[r, t2] = cfg.eos_id
    return tok


def _rewards(cfg: Config) -> np.ndarray:
    N, G = cfg.N, cfg.G
    if cfg.reward == "bernoulli":
        return (uniform01(cfg.seed, S_REWARDS, np.arange(N)) < cfg.p).astype(np.float32)
    if cfg.reward == "graded":
        return (randint(cfg.seed, S_REWARDS, np.arange(N), 5).astype(np.float32) / 4.0)
    if cfg.reward == "tiny":
        out = np.empty(N, dtype=np.float32)
        out[:G] = 1.0
        for b in range(1, cfg.B):
            attempt = 0
            while True:
                ctr = (b * 1000 + attempt) * G + np.arange(G)
                r = (uniform01(cfg.seed, S_REWARDS, ctr) < cfg.p).astype(np.float32)
                if r.min() != r.max():
                    break
                attempt += 1
            out[b * G:(b + 1) * G] = r
        return out
    raise ValueError(cfg.reward)


def make_case(cfg: Config) -> Case:
    N, C = cfg.N, cfg.C
    old = normal64(cfg.seed, S_OLD_NOISE, np.arange(N * C), cfg.old_noise).reshape(N, C)
    ref = None
    if cfg.ref_noise is not None:
        ref = normal64(cfg.seed, S_REF_NOISE, np.arange(N * C), cfg.ref_noise).reshape(N, C)
    return Case(cfg=cfg, tokens=_tokens(cfg), rewards=_rewards(cfg), old_noise=old,
                ref_noise=ref)


def perturb(logp: np.ndarray, noise: np.ndarray) -> np.ndarray:
    """float32(logp + noise): an 'old' or 'reference' log-prob near logp."""
    return (np.asarray(logp, dtype=np.float64) + noise).astype(np.float32)
